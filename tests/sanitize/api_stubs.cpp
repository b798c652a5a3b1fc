// Host-only stand-ins for the device-side launchers of libgq, so that the C
// ABI layer (csrc/gq_api.cpp: argument checks, table planning, workspace
// layout) can be built and run under host sanitizers without a GPU.  Every
// launcher counts its calls and returns success; the shape helpers return
// fixed, plausible values.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "gq_internal.h"

int g_launches = 0;

namespace gq {

namespace {
hipError_t launch() { ++g_launches; return hipSuccess; }
float g_scratch[16];
} // namespace

int device_cus() { return 256; }
hipError_t launch_dequant_q8_0(const void *, float *, uint16_t *, int64_t, int64_t, hipStream_t) { return launch(); }
hipError_t launch_dequant_q4k(const void *, float *, uint16_t *, int64_t, int64_t, hipStream_t) { return launch(); }
hipError_t launch_gemv_q8_0(const void *, const float *, float *, int64_t, int64_t, int, hipStream_t) { return launch(); }
hipError_t launch_gemv_q4k(const void *, const float *, float *, int64_t, int64_t, int, hipStream_t) { return launch(); }
long long gemv_stream_tiles(int64_t M, int64_t) { return (M + 23) / 24; }
int gemv_stream_grid(long long, long long tiles) { return tiles < 512 ? (int)tiles : 512; }
hipError_t launch_gemv_stream(const GemvEntry *, const GemvEntry &, int, long long, int, hipStream_t) { return launch(); }
hipError_t launch_gemv_swiglu(const void *, const void *, const float *, float *, int64_t, int64_t, hipStream_t) { return launch(); }
long long gemv_mfma_blocks(int64_t M, int tiles) { return (M + 64 * tiles - 1) / (64 * tiles); }
hipError_t launch_gemv_mfma(const GemvEntry *, const GemvEntry &, int, long long, long long, long long, long long, int, hipStream_t) { return launch(); }
long long gemv_mfma_prestaged_bytes(int64_t n, long long records, int B) { return gemv_prestaged_records_offset(n) + records * 1024 * ((608 + 1024 * B + 1023) / 1024); }
hipError_t launch_gemv_mfma_prestaged(const GemvEntry *, int, long long, long long, long long, long long, long long, int, void *, hipStream_t) { return launch(); }
hipError_t launch_gemv_swiglu_mfma(const void *, const void *, const float *, float *, int64_t, int64_t, int, hipStream_t) { return launch(); }
hipError_t launch_gemm_q4k(const void *, const uint16_t *, uint16_t *, int64_t, int64_t, int64_t, hipStream_t) { return launch(); }
hipError_t launch_gemm_q8_0(const void *, const uint16_t *, uint16_t *, int64_t, int64_t, int64_t, hipStream_t) { return launch(); }
bool gemm_big_fits(int64_t, int64_t K, int64_t N) { return N * K * 2 < ((int64_t)1 << 31); }
int gemm_big_choice(int64_t, int64_t, int64_t) { return 256; }
int gemm_kgroups_choice(int64_t, int64_t K, int64_t N) { return N < 256 && (K / 256) % 4 == 0 ? 4 : 0; }
hipError_t launch_gemm_kgroups(const void *, const uint16_t *, uint16_t *, int64_t, int64_t, int64_t, int, bool, hipStream_t) { return launch(); }
hipError_t launch_gemm_big(const void *, const uint16_t *, uint16_t *, int64_t, int64_t, int64_t, int, bool, hipStream_t) { return launch(); }
int gemm_splitk_choice(int64_t, int64_t K, int64_t) { return (K / 256) % 2 == 0 ? 2 : 1; }
hipError_t launch_gemm_splitk(const void *, const uint16_t *, uint16_t *, int64_t, int64_t, int64_t, int, float *, hipStream_t) { return launch(); }
hipError_t splitk_scratch(float **out) { *out = g_scratch; return hipSuccess; }
hipError_t launch_moe(const MoeArgs &, hipStream_t) { return launch(); }
hipError_t launch_gemv_q8_0_mfma(const void *, const float *, float *, int64_t, int64_t, int, hipStream_t) { return launch(); }
hipError_t launch_gemv_q4k_f32(const void *, const float *, float *, int64_t, int64_t, int, hipStream_t) { return launch(); }
hipError_t launch_quantize_q8k(const float *, int8_t *, float *, int32_t *, int64_t, int64_t, hipStream_t) { return launch(); }
hipError_t launch_gemv_q4k_q8k(const void *, const int8_t *, const float *, const int32_t *, float *, int64_t, int64_t, int, hipStream_t) { return launch(); }
hipError_t launch_gemm_q4k_q8k(const void *, const int8_t *, const float *, float *, int64_t, int64_t, int64_t, hipStream_t) { return launch(); }
hipError_t launch_moe_route(const float *, int32_t *, float *, int64_t, int64_t, int64_t, bool, hipStream_t) { return launch(); }
int moe_token_tile(int64_t, int64_t) { return 128; }
bool moe_skinny_applies(int64_t, int64_t) { return false; }
hipError_t launch_moe_skinny(const MoeArgs &, hipStream_t) { return launch(); }
bool moe_big_applies(int64_t, int64_t, int64_t, int64_t) { return false; }
int moe_big_token_tile() { return 256; }
hipError_t launch_moe_big(const MoeArgs &, int, hipStream_t) { return launch(); }

} // namespace gq
