// dsa_phase.hpp -- optional phase timestamps for the decode-step kernels.
//
// Built only into the trace library (build.py --trace defines DSA_PHASE_TRACE); in the product
// library every marker below compiles to nothing. With it, thread 0 of a block stores the
// 100 MHz constant clock (s_memrealtime) at a named point of its kernel into a device table of
// the translation unit (each .hip file is its own code object), and an extern "C" reader
// copies the table to the host. The tables keep the stamps of the last launch of each kernel:
// phase_trace.py launches each kernel of one step, reads the tables and summarises them.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {
namespace phase {
// kernel: 0 compact_index_scores, 1 topk_expand, 2 sparse MLA main, 3 MLA combine.
constexpr int kKernels = 4;
constexpr int kBlocks = 4096;  // linear block ids past this are not recorded
constexpr int kSlots = 8;
constexpr size_t kTableBytes = sizeof(unsigned long long) * kKernels * kBlocks * kSlots;
}  // namespace phase
}  // namespace dsa

#ifdef DSA_PHASE_TRACE

// One table per translation unit, with its reader dsa_phase_read_<name>(host buffer of
// kTableBytes) and dsa_phase_clear_<name>() (zeroes it), which return the HIP status. Both
// synchronise with the device; they are for the trace tool, never for a captured stream.
#define DSA_PHASE_TABLE(name)                                                                    \
    namespace dsa {                                                                              \
    namespace phase {                                                                            \
    static __device__ unsigned long long table[kKernels * kBlocks * kSlots];                     \
    }                                                                                            \
    }                                                                                            \
    extern "C" int dsa_phase_read_##name(void *dst) {                                            \
        return (int)hipMemcpyFromSymbol(dst, HIP_SYMBOL(dsa::phase::table), dsa::phase::kTableBytes, \
                                        0, hipMemcpyDeviceToHost);                               \
    }                                                                                            \
    extern "C" int dsa_phase_clear_##name() {                                                    \
        static const unsigned long long zeros[dsa::phase::kKernels * dsa::phase::kBlocks *       \
                                              dsa::phase::kSlots] = {};                          \
        return (int)hipMemcpyToSymbol(HIP_SYMBOL(dsa::phase::table), zeros, dsa::phase::kTableBytes, \
                                      0, hipMemcpyHostToDevice);                                 \
    }

// Stamp `slot` of kernel `k` for this block (thread 0 only; an ordinary global store).
#define DSA_PHASE(k, slot)                                                                       \
    do {                                                                                         \
        if (threadIdx.x == 0) {                                                                  \
            const int b_ = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);       \
            if (b_ < ::dsa::phase::kBlocks)                                                      \
                ::dsa::phase::table[((k) * ::dsa::phase::kBlocks + b_) * ::dsa::phase::kSlots +  \
                                    (slot)] = __builtin_amdgcn_s_memrealtime();                  \
        }                                                                                        \
    } while (0)

#else

#define DSA_PHASE_TABLE(name)
#define DSA_PHASE(k, slot) \
    do {                   \
    } while (0)

#endif
