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

  if (step_copy_role<DT, D, BS, NT>(a, a.num_seqs * (a.num_kv_heads / a.heads_per_wg))) return;
  Row st;
  PartitionWork w;
  if (!partition_prologue<DT, D, BS, G, NT>(a, lane, w, [&](int b, int gg) {
        const int g = gg * hpw + hw;
        st.load_q(static_cast<const S*>(a.q) + ((size_t)b * a.num_q_heads + g * G + hs * GW) * D,
                  col);
      }))
    return;
  const int g = w.gg * hpw + hw;
  const int ctx = w.ctx, blk0 = w.blk0;

  st.reset();
  // A block's rows through buffer loads over that block: 16 bytes a lane at
  // d = E col of token t ROWS + row.  The resource covers the block's rows
  // below the context length only, so the rows past it in a sequence's last
  // block read nothing (they return zeros, and are masked anyway); the
  // prefetch past a wave's last block (live false) gets a resource of zero
  // bytes, so it reads nothing instead of the last block once more.
  constexpr int ROWS = Sh::ROWS;
  const uint32_t tok_bytes = (uint32_t)((size_t)Hkv * D * sizeof(S));
  const uint32_t blk_bytes = tok_bytes * BS;
  const uint32_t lane_bytes = (uint32_t)(((size_t)row * Hkv * D + (size_t)g * D + col * E) * sizeof(S));
  const char* kbase = static_cast<const char*>(a.k_cache);
  const char* vbase = static_cast<const char*>(a.v_cache);
  auto fetch = [&](int j, bool live, uint4 (&kr)[NI], uint4 (&vr)[NI]) {
    const size_t off = (size_t)w.block(j) * blk_bytes;
    const int rows = min(BS, ctx - (blk0 + j) * BS);  // >= 1 for a live block
    const uint32_t n = live ? (uint32_t)rows * tok_bytes : 0u;
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(kbase + off), 0, n, kBufferWord3);
    const __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(vbase + off), 0, n, kBufferWord3);
#pragma unroll
    for (int t = 0; t < NI; ++t)
      kr[t] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                            rk, lane_bytes + t * ROWS * tok_bytes, 0, kLoadNT));
#pragma unroll
    for (int t = 0; t < NI; ++t)
      vr[t] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                            rv, lane_bytes + t * ROWS * tok_bytes, 0, kLoadNT));
  };
  // A decode step's new token (position ctx - 1, in the last partition):
  // the wave that folds its block takes the step's K/V rows in place of what
  // it read in that slot (the copy workgroups store them).  Rows past the
  // context load the block's token 0, which is that slot when the new token
  // opens its block (tt == 0): they take the new rows too, so that no stale
  // value -- uninitialised memory, NaN included -- reaches a masked product.
  const bool step = a.new_k != nullptr && w.part == w.nparts - 1;
  const int tj = step ? (ctx - 1) / BS - blk0 : -1;  // block of the new token
  const int tt = (ctx - 1) % BS, tli = tt / ROWS, tlr = tt % ROWS;
  uint4 nk = make_uint4(0, 0, 0, 0), nv = nk;
  if (step) {
    const size_t src = ((size_t)w.b * Hkv + g) * D + col * E;
    nk = load_chunk(static_cast<const S*>(a.new_k) + src);
    nv = load_chunk(static_cast<const S*>(a.new_v) + src);
  }
  auto consume = [&](int j, bool live, uint4 (&kr)[NI], uint4 (&vr)[NI]) {
    if (j == tj) {
#pragma unroll
      for (int ii = 0; ii < NI; ++ii) {
        if (tt == 0 || (ii == tli && row == tlr)) {
          kr[ii] = nk;
          vr[ii] = nv;
        }
      }
    }
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

template <class DT, int D, int G>
__global__ __launch_bounds__(D) void merge_partitions_kernel(DecodeArgs a, int bs) {
  merge_partitions<DT, D, G>(a, bs);
}

template <class DT, int D, int BS, int G>
hipError_t launch_partition_t(const DecodeArgs& a, hipStream_t stream) {
  constexpr int NT = kDecodeWaves * 64;
  const int copy_wgs = step_copy_workgroups(a, D, sizeof(typename DT::storage), NT);
  dim3 grid(a.num_seqs * (a.num_kv_heads / a.heads_per_wg) + copy_wgs, a.max_parts);
  decode_partition_kernel<DT, D, BS, G, kDecodeWaves><<<grid, kDecodeWaves * 64, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_merge(int dtype, int D, int BS, int G, const DecodeArgs& a, hipStream_t s) {
  return dispatch_decode(dtype, D, 16, G, [&](auto dt, auto d, auto, auto g) {
    constexpr int Dv = decltype(d)::value;
    merge_partitions_kernel<decltype(dt), Dv, decltype(g)::value>
        <<<a.num_seqs * a.num_q_heads, Dv, 0, s>>>(a, BS);
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
