// Measurement build only (PA_TIMELINE defined; never in the library's
// default build): every worker wave of a stream kernel records, for the
// latest launch, the GPU's constant clock at its start, once its first block
// is requested (end of the prologue), at the end of its range (end of the
// stream) and when it is done (after its merge, if it merges), with its
// hardware ids and whether it merged.  Each kernel source that includes this
// header keeps its own record array; PA_TIMELINE_READER(name) defines the
// C function that copies that source's records to the host.  Without
// PA_TIMELINE the stamps compile to nothing.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

namespace pa {

#ifdef PA_TIMELINE
constexpr int kTimelineWaves = 16384;
// t_start, t_prologue, t_stream, t_done, hw ids, pieces merged, t_lengths (prefix
// sum of the lengths done), t_range (range's table entries requested)
constexpr int kTimelineWords = 8;
static __device__ unsigned long long pa_timeline[kTimelineWaves * kTimelineWords];
struct WaveStamps {
  unsigned long long* rec;
  __device__ explicit WaveStamps(int global_wave)
      : rec(global_wave < kTimelineWaves ? pa_timeline + (size_t)global_wave * kTimelineWords
                                         : nullptr) {}
  __device__ void put(int k, unsigned long long v) const {
    if (rec && (threadIdx.x & 63) == 0) rec[k] = v;
  }
  __device__ void now(int k) const { put(k, __builtin_amdgcn_s_memrealtime()); }
  // HW_ID (wave, SIMD, CU, shader array, engine) and, above bit 32, XCC_ID.
  __device__ void ids() const {
    put(4, (unsigned long long)__builtin_amdgcn_s_getreg((31 << 11) | 4) |
               ((unsigned long long)__builtin_amdgcn_s_getreg((3 << 11) | 20) << 32));
  }
};
#define PA_STAMP(obj, k) (obj).now(k)
#define PA_STAMP_IDS(obj) (obj).ids()
#define PA_STAMP_VALUE(obj, k, v) (obj).put(k, v)
// Copy this source's records on the current device to host memory (entries
// of kTimelineWords words), then clear them, and report the constant clock's
// frequency in kHz.  Read once, run one launch, read again: the second read
// holds that launch's waves and zeros elsewhere.  Returns the words copied,
// or -1.
#define PA_TIMELINE_READER(name)                                                          \
  extern "C" int32_t name(unsigned long long* host, int64_t max_words, int32_t* clock_khz) { \
    void* p = nullptr;                                                                    \
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(pa::pa_timeline)) != hipSuccess) return -1;   \
    const int64_t words = (int64_t)pa::kTimelineWaves * pa::kTimelineWords;              \
    const int64_t n = max_words < words ? max_words : words;                              \
    if (hipDeviceSynchronize() != hipSuccess) return -1;                                  \
    if (hipMemcpy(host, p, (size_t)n * 8, hipMemcpyDeviceToHost) != hipSuccess) return -1; \
    if (hipMemset(p, 0, (size_t)words * 8) != hipSuccess) return -1;                      \
    if (hipDeviceSynchronize() != hipSuccess) return -1;                                  \
    int dev = 0, khz = 0;                                                                 \
    if (hipGetDevice(&dev) != hipSuccess ||                                               \
        hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess)  \
      return -1;                                                                          \
    *clock_khz = khz;                                                                     \
    return (int32_t)n;                                                                    \
  }
#else
struct WaveStamps {
  __device__ explicit WaveStamps(int) {}
};
#define PA_STAMP(obj, k) ((void)0)
#define PA_STAMP_IDS(obj) ((void)0)
#define PA_STAMP_VALUE(obj, k, v) ((void)0)
#define PA_TIMELINE_READER(name)
#endif

}  // namespace pa
