// Launch plumbing shared by the decode kernels: template dispatch over the
// built shapes and the per-kernel launchers.
#pragma once

#include "attn_common.hpp"

namespace pa {

#ifndef PA_DECODE_WAVES
#define PA_DECODE_WAVES 4
#endif
constexpr int kDecodeWaves = PA_DECODE_WAVES;  // waves per workgroup

// Calls f(dtype_tag, IntC<D>, IntC<BS>, IntC<G>) for the built combination.
template <class F>
hipError_t dispatch_decode(int dtype, int D, int BS, int G, F&& f) {
  auto by_g = [&](auto dt, auto d, auto bs) -> hipError_t {
    switch (G) {
      case 1: return f(dt, d, bs, IntC<1>{});
      case 2: return f(dt, d, bs, IntC<2>{});
      case 4: return f(dt, d, bs, IntC<4>{});
      case 8: return f(dt, d, bs, IntC<8>{});
      case 16: return f(dt, d, bs, IntC<16>{});
      case 32: return f(dt, d, bs, IntC<32>{});
    }
    return hipErrorInvalidValue;
  };
  auto by_bs = [&](auto dt, auto d) -> hipError_t {
    return BS == 16 ? by_g(dt, d, IntC<16>{}) : by_g(dt, d, IntC<32>{});
  };
  auto by_d = [&](auto dt) -> hipError_t {
    return D == 64 ? by_bs(dt, IntC<64>{}) : by_bs(dt, IntC<128>{});
  };
  return dtype == PA_DTYPE_BF16 ? by_d(BF16{}) : by_d(F32{});
}

hipError_t launch_partition(int dtype, int D, int BS, int G, const DecodeArgs& a,
                            hipStream_t s);

// Matrix-core kernel for query groups of 4 or more (bfloat16, G in {4, 8, 16, 32}):
// same arguments, workspace and results as launch_partition.
bool mfma_supported(int dtype, int D, int BS, int G);
hipError_t launch_mfma(int D, int BS, int G, const DecodeArgs& a, hipStream_t s);

constexpr int kStreamWaves = 4;  // worker waves per workgroup of the stream schedule
// Waves per workgroup of the stream schedule's matrix-core worker: 8 at
// head_dim 64, where a workgroup of eight fits the registers and LDS (the
// Llama-3.2-shaped batch: 50.5 against 51.9 us with four), 4 at head_dim 128.
__host__ __device__ constexpr int stream_mfma_waves(int D) { return D == 64 ? 8 : 4; }
// Worker counts per kv head are rounded to a multiple of this, so that every
// workgroup of either worker holds whole ranges.
constexpr int kStreamRangeQuantum = 8;

// Kv heads one stream workgroup takes (one wave each, over kStreamWaves / HW
// consecutive ranges): as many as divide both the waves and the kv heads.
__host__ __device__ inline int stream_heads_per_wg(int Hkv) {
  return Hkv % 4 == 0 ? 4 : Hkv % 2 == 0 ? 2 : 1;
}

// Balanced schedule (decode_stream.hip): worker waves over equal ranges of
// each kv head's block list, G in {1, 2, 4}; same workspace contract.
bool stream_supported(int G);
hipError_t launch_stream(int dtype, int D, int BS, int G, const DecodeArgs& a, hipStream_t s);
// The balanced schedule's matrix-core worker (decode_stream_mfma.hip):
// bfloat16, G = 4.  Same ranges, workspace and merge as launch_stream.
bool stream_mfma_supported(int dtype, int G);
hipError_t launch_stream_mfma(int D, int BS, int G, const DecodeArgs& a, hipStream_t s);
// Merge kernel run after a stream launch with deferred_merge set.
hipError_t launch_stream_merge(int dtype, int D, int BS, int G, const DecodeArgs& a,
                               hipStream_t s);

// Merge kernel run after a partition launch with deferred_merge set.
hipError_t launch_merge(int dtype, int D, int BS, int G, const DecodeArgs& a, hipStream_t s);


}  // namespace pa
