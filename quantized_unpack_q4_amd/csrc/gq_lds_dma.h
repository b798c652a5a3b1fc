// gq_lds_dma.h -- direct global -> LDS copies for the gfx950 kernels of libgq.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gq {

// 16 bytes per lane, global -> LDS: lane l reads gbase + voff (gbase
// wave-uniform, voff a 32-bit byte offset) and lands at LDS byte address
// m0 + 16*l (m0 wave-uniform).  Issued as inline assembly so that the
// compiler's wait insertion does not see it: a kernel waits for these copies
// itself, with an explicit vmcnt before the barrier that publishes them.  The
// compiler then counts fewer outstanding loads than there are, so every wait
// it inserts for its own loads errs on the safe side.
__device__ __forceinline__ void load_lds16(const void *gbase, uint32_t voff, uint32_t m0)
{
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(gbase),
                 "s"(m0)
                 : "memory", "m0");
}

} // namespace gq
