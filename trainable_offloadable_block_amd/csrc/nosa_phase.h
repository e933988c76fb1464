// Phase clocks of the timing build of the library (compiled with
// -DNOSA_PHASE_CLOCKS; the default build stamps nothing): thread 0 of a
// workgroup (or lane 0 of a wave) writes the GPU's constant 100 MHz
// real-time counter at phase boundaries into a per-source-file device array
// [pair][row][slot], which the timing build's nosa_phase_clocks_* calls copy
// out. Used to break a launch's time into its phases.
#pragma once

#ifdef NOSA_PHASE_CLOCKS
namespace nosa {
constexpr int kPhasePairs = 512, kPhaseRows = 40, kPhaseSlots = 16;
constexpr int kPhasePoolRow = kPhaseRows - 1;   // the pair's last workgroup's own phases
}  // namespace nosa
static __device__ unsigned long long
    g_phase_clock[nosa::kPhasePairs * nosa::kPhaseRows * nosa::kPhaseSlots];
#define NOSA_PHASE_AT(cond, p, row, slot)                                                  \
  do {                                                                                     \
    if ((cond) && (p) < nosa::kPhasePairs && (row) < nosa::kPhaseRows)                     \
      g_phase_clock[((p) * nosa::kPhaseRows + (row)) * nosa::kPhaseSlots + (slot)] =       \
          __builtin_amdgcn_s_memrealtime();                                                \
  } while (0)
#define NOSA_PHASE(p, row, slot) NOSA_PHASE_AT(threadIdx.x == 0, p, row, slot)
// Stores a value (a count) rather than the clock.
#define NOSA_PHASE_VAL(p, row, slot, val)                                                  \
  do {                                                                                     \
    if (threadIdx.x == 0 && (p) < nosa::kPhasePairs && (row) < nosa::kPhaseRows)           \
      g_phase_clock[((p) * nosa::kPhaseRows + (row)) * nosa::kPhaseSlots + (slot)] =       \
          (unsigned long long)(val);                                                       \
  } while (0)
#define NOSA_PHASE_WAVE(p, row, slot) NOSA_PHASE_AT((threadIdx.x & 63) == 0, p, row, slot)
// Copies the array out (dst, when not NULL), then zeroes it (when clear).
#define NOSA_PHASE_READER(name)                                                            \
  extern "C" int name(void *dst, size_t bytes, int clear) {                                \
    if (dst && hipMemcpyFromSymbol(dst, HIP_SYMBOL(g_phase_clock), bytes) != hipSuccess)   \
      return -5;                                                                           \
    if (clear) {                                                                           \
      static unsigned long long zeros[sizeof(g_phase_clock) / 8];                          \
      if (hipMemcpyToSymbol(HIP_SYMBOL(g_phase_clock), zeros, sizeof(zeros)) != hipSuccess) \
        return -5;                                                                         \
    }                                                                                      \
    return 0;                                                                              \
  }
#else
#define NOSA_PHASE(p, row, slot) \
  do {                           \
  } while (0)
#define NOSA_PHASE_WAVE(p, row, slot) \
  do {                                \
  } while (0)
#define NOSA_PHASE_VAL(p, row, slot, val) \
  do {                                    \
  } while (0)
#endif
