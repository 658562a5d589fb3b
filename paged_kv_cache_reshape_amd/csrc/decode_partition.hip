// Decode attention, fixed-size partitions: one workgroup per (kv-head group,
// sequence, partition of part_blocks logical blocks).
//
//   * a workgroup takes hpw consecutive kv heads (their rows are neighbours in
//     every token) and all G query heads of each; every K/V byte is fetched
//     from HBM once per (sequence, kv head);
//   * the partition's block-table entries are read with two vector loads
//     (lane l holds entries l and 64 + l) and broadcast with readlane;
//   * a sequence longer than one partition leaves one partial state per
//     partition; the last workgroup of that (sequence, head group) to arrive
//     merges them in the same launch (the last-block pattern of the LLAISYS
//     README, CUDA argmax item).  Used when the caller fixes the partition
//     size (the long-context workload states 512 tokens).
#include "attn_common.hpp"

#include "decode_launch.hpp"

namespace pa {

template <class DT, int D, int BS, int G, int NW>
__global__ __launch_bounds__(NW * 64) void decode_partition_kernel(DecodeArgs a) {
  using Sh = DecodeShape<DT, D, BS, G, NW>;
  using Row = RowAttn<DT, D, BS, G, NW>;
  using S = typename DT::storage;
  constexpr int E = Sh::E, RL = Sh::RL, NI = Sh::NI;
  constexpr int GW = Sh::GW, HS = Sh::HS;
  constexpr int NT = NW * 64;

  const int hpw = a.heads_per_wg;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keep loops scalar
  const int Hkv = a.num_kv_heads;
  const int nwt = NW / (hpw * HS);  // waves sharing one (kv head, head slice)

  // Wave roles: kv head of the group, slice of its query heads, token split.
  const int hw = wave % hpw;
  const int hs = (wave / hpw) % HS;
  const int tw = wave / (hpw * HS);
  const int row = lane / RL;
  const int col = lane % RL;

  Row st;
  PartitionWork w;
  if (!partition_prologue<DT, D, BS, G, NT>(a, lane, w, [&](int b, int gg) {
        const int g = gg * hpw + hw;
        st.load_q(static_cast<const S*>(a.q) + ((size_t)b * a.num_q_heads + g * G + hs * GW) * D,
                  col);
      }))
    return;
  if (a.new_k != nullptr && w.part == w.nparts - 1) write_step_token<DT, D, BS, NT>(a, w);
  const int g = w.gg * hpw + hw;
  const int ctx = w.ctx, blk0 = w.blk0;

  st.reset();
  const size_t tok_stride = (size_t)Hkv * D;
  const size_t blk_stride = tok_stride * BS;
  const int lane_off = row * Hkv * D + col * E;
  const S* kbase = static_cast<const S*>(a.k_cache) + (size_t)g * D + lane_off;
  const S* vbase = static_cast<const S*>(a.v_cache) + (size_t)g * D + lane_off;
  auto fetch = [&](int j, uint4 (&kr)[NI], uint4 (&vr)[NI]) {
    const size_t off = (size_t)w.block(j) * blk_stride;
    Row::fetch(kbase + off, vbase + off, tok_stride, kr, vr);
  };
  auto consume = [&](int j, bool live, const uint4 (&kr)[NI], const uint4 (&vr)[NI]) {
    st.consume((blk0 + j) * BS + row, ctx, live, a.scale_log2, kr, vr);
  };
  stream_blocks<NI>(tw, nwt, w.nblk_run, fetch, consume);
  st.merge_rows();

  __shared__ __attribute__((aligned(16))) float s_acc[NW][GW][D];
  __shared__ float s_m[NW][GW];
  __shared__ float s_l[NW][GW];
  st.to_lds(s_acc[wave], s_m[wave], s_l[wave], lane);
  __syncthreads();
  finish_partition<DT, D, G, GW, HS, NW, NW / HS>(a, w.b, w.gg, w.part, w.nparts,
                                                  w.poisoned, s_acc, s_m, s_l);
}

template <class DT, int D, int G, int NT>
__global__ __launch_bounds__(NT) void merge_partitions_kernel(DecodeArgs a, int bs) {
  merge_partitions<DT, D, G, NT>(a, bs);
}

template <class DT, int D, int BS, int G>
hipError_t launch_partition_t(const DecodeArgs& a, hipStream_t stream) {
  dim3 grid(a.num_seqs * (a.num_kv_heads / a.heads_per_wg), a.max_parts);
  decode_partition_kernel<DT, D, BS, G, kDecodeWaves><<<grid, kDecodeWaves * 64, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_merge(int dtype, int D, int BS, int G, const DecodeArgs& a, hipStream_t s) {
  return dispatch_decode(dtype, D, 16, G, [&](auto dt, auto d, auto, auto g) {
    merge_partitions_kernel<decltype(dt), decltype(d)::value, decltype(g)::value, 256>
        <<<a.num_seqs * a.num_kv_heads, 256, 0, s>>>(a, BS);
    return hipGetLastError();
  });
}

hipError_t launch_partition(int dtype, int D, int BS, int G, const DecodeArgs& a,
                            hipStream_t s) {
  return dispatch_decode(dtype, D, BS, G, [&](auto dt, auto d, auto bs, auto g) {
    return launch_partition_t<decltype(dt), decltype(d)::value, decltype(bs)::value,
                              decltype(g)::value>(a, s);
  });
}

}  // namespace pa
