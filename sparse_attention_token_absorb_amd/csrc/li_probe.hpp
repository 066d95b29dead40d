// Phase timestamps of the decode scoring kernels: instrumentation compiled
// only into the "phases" build variant (LI_PHASE_PROBE defined); in the
// product build every macro here expands to nothing.
//
// Each wave of a decode scoring launch records five readings of the 100 MHz
// constant clock (s_memrealtime): its start, the moment its first tile of
// latent rows has landed in LDS, the end of its stream, the end of the
// workgroup barrier after the stream, and its end.  Lane 0 stores them with
// the wave's XCC id, hardware id and workgroup coordinates, eight 64-bit
// words per wave, indexed by (blockIdx.y * gridDim.x + blockIdx.x) * 4 + wave.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace li {

constexpr int kProbeWaves = 16384; // waves recorded per launch (later ones are not)
constexpr int kProbeWords = 8;     // 64-bit words per wave record

#ifdef LI_PHASE_PROBE

#define LI_PHASE_DECL uint64_t li_ph0 = 0, li_ph1 = 0, li_ph2 = 0, li_ph3 = 0, li_ph4 = 0
#define LI_PHASE(var) asm volatile("s_memrealtime %0\n\ts_waitcnt lgkmcnt(0)" : "=s"(var))
#define LI_PHASE_START LI_PHASE(li_ph0)
#define LI_PHASE_FIRST_IF(cond) \
    if (cond) LI_PHASE(li_ph1)
#define LI_PHASE_LOOP LI_PHASE(li_ph2)
#define LI_PHASE_SYNC LI_PHASE(li_ph3)
#define LI_PHASE_STORE(buf, wave, lane)                                                                             \
    do {                                                                                                           \
        LI_PHASE(li_ph4);                                                                                          \
        const int64_t li_slot = ((int64_t)blockIdx.y * gridDim.x + blockIdx.x) * 4 + (wave);                       \
        if ((lane) == 0 && li_slot < kProbeWaves) {                                                                \
            uint64_t *li_d = (buf) + li_slot * kProbeWords;                                                        \
            li_d[0] = li_ph0;                                                                                      \
            li_d[1] = li_ph1;                                                                                      \
            li_d[2] = li_ph2;                                                                                      \
            li_d[3] = li_ph3;                                                                                      \
            li_d[4] = li_ph4;                                                                                      \
            /* XCC_ID (hwreg 20, 16 bits) and HW_ID (hwreg 4) */                                                   \
            li_d[5] = ((uint64_t)__builtin_amdgcn_s_getreg(30740) << 32) | (uint32_t)__builtin_amdgcn_s_getreg(63492); \
            li_d[6] = blockIdx.x;                                                                                  \
            li_d[7] = blockIdx.y;                                                                                  \
        }                                                                                                          \
    } while (0)

#else

#define LI_PHASE_DECL
#define LI_PHASE_START
#define LI_PHASE_FIRST_IF(cond)
#define LI_PHASE_LOOP
#define LI_PHASE_SYNC
#define LI_PHASE_STORE(buf, wave, lane)

#endif

// Host side: the device address of one kernel's records on the current
// device (bf16 decode scoring in score.hip, FP8 decode scoring in fp8.hip);
// hipErrorNotSupported in the product build.
hipError_t phase_records_bf16(void **dev);
hipError_t phase_records_fp8(void **dev);

} // namespace li
