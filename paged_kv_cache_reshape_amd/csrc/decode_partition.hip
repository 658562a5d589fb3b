// Decode attention, fixed-size partitions: one workgroup per (kv-head group,
// sequence, partition of part_blocks logical blocks).
//
//   * a workgroup takes hpw consecutive kv heads (their rows are neighbours in
//     every token) and all G query heads of each; every K/V byte is fetched
//     from HBM once per (sequence, kv head);
//   * the partition's block-table entries are read with one vector load (lane
//     j holds entry j) and broadcast with readlane;
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
  constexpr int GW = Sh::GW, HS = Sh::HS, GH = Sh::GH;
  constexpr int NT = NW * 64;

  // Grid: x = (kv-head group, sequence), y = partition.  Workgroups are dealt
  // to the XCDs round-robin in linear-id order; with the partition index
  // slowest every partition index is spread over all XCDs (with it fastest,
  // partition p of every sequence would land on XCD p mod 8).
  const int hpw = a.heads_per_wg;
  const int n_groups = a.num_kv_heads / hpw;
  const int gg = blockIdx.x % n_groups;
  const int b = blockIdx.x / n_groups;
  const int part = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keep loops scalar
  const int Hkv = a.num_kv_heads;
  const int nwt = NW / (hpw * HS);  // waves sharing one (kv head, head slice)

  // Wave roles: kv head of the group, slice of its query heads, token split.
  const int hw = wave % hpw;
  const int hs = (wave / hpw) % HS;
  const int tw = wave / (hpw * HS);
  const int g = gg * hpw + hw;
  const int row = lane / RL;
  const int col = lane % RL;

  // Everything the first K/V load depends on is requested together.
  const int ctx = a.context_lens[b];
  const int blk0 = part * a.part_blocks;
  const int32_t* trow = a.block_tables + (size_t)b * a.max_blocks + blk0;
  const int my_blk =
      (lane < a.part_blocks && blk0 + lane < a.max_blocks) ? trow[lane] : 0;
  Row st;
  st.load_q(static_cast<const S*>(a.q) + ((size_t)b * a.num_q_heads + g * G + hs * GW) * D,
            col);

  const int part_tokens = a.part_blocks * BS;
  const bool bad_ctx = ctx < 0 || ctx > a.max_blocks * BS;
  const int nparts = (bad_ctx || ctx == 0) ? 1 : (ctx + part_tokens - 1) / part_tokens;
  if (part >= nparts) return;

  const int wg_elems = hpw * G * D;
  const size_t out_base = ((size_t)b * a.num_q_heads + (size_t)gg * hpw * G) * D;
  if (bad_ctx || ctx == 0) {
    const float fill = bad_ctx ? __builtin_nanf("") : 0.0f;
    for (int e = tid; e < wg_elems; e += NT) store_out(DT{}, a.out, out_base + e, fill);
    return;
  }

  const int nblk_seq = (ctx + BS - 1) / BS;
  const int nblk = min(a.part_blocks, nblk_seq - blk0);
  const bool bad_here = lane < nblk && (my_blk < 0 || my_blk >= a.num_blocks);
  const bool poisoned = __ballot(bad_here) != 0;  // same answer in every wave
  const int nblk_run = poisoned ? 0 : nblk;

  st.reset();
  const size_t tok_stride = (size_t)Hkv * D;
  const size_t blk_stride = tok_stride * BS;
  const int lane_off = row * Hkv * D + col * E;
  const S* kbase = static_cast<const S*>(a.k_cache) + (size_t)g * D + lane_off;
  const S* vbase = static_cast<const S*>(a.v_cache) + (size_t)g * D + lane_off;
  auto fetch = [&](int j, uint4 (&kr)[NI], uint4 (&vr)[NI]) {
    const size_t off = (size_t)__builtin_amdgcn_readlane(my_blk, j) * blk_stride;
    Row::fetch(kbase + off, vbase + off, tok_stride, kr, vr);
  };
  auto consume = [&](int j, bool live, const uint4 (&kr)[NI], const uint4 (&vr)[NI]) {
    st.consume((blk0 + j) * BS + row, ctx, live, a.scale_log2, kr, vr);
  };
  // Two blocks in flight per wave.
  stream_blocks<NI>(tw, nwt, nblk_run, fetch, consume);
  st.merge_rows();

  __shared__ float s_acc[NW][GW][D];
  __shared__ float s_m[NW][GW];
  __shared__ float s_l[NW][GW];
  __shared__ int s_last;
  st.to_lds(s_acc[wave], s_m[wave], s_l[wave], lane);
  __syncthreads();

  // Waves on one (kv head, head slice) -> the partition's state per element.
  for (int e = tid; e < wg_elems; e += NT) {
    const int hwe = e / (G * D), rem = e % (G * D);
    const int hh = rem / D, d = rem % D;
    const int w0 = hwe + hpw * (hh / GW);
    const int h = hh % GW;
    float M = kNoMax;
    for (int t = 0; t < nwt; ++t) M = fmaxf(M, s_m[w0 + hpw * HS * t][h]);
    float L = 0.0f, A = 0.0f;
    for (int t = 0; t < nwt; ++t) {
      const int w = w0 + hpw * HS * t;
      const float f = fast_exp2(s_m[w][h] - M);
      L += s_l[w][h] * f;
      A += s_acc[w][h][d] * f;
    }
    if (poisoned) L = __builtin_nanf("");
    if (nparts == 1) {
      store_out(DT{}, a.out, out_base + e, A / L);
    } else {
      const size_t pr = (((size_t)b * Hkv + gg * hpw + hwe) * a.max_parts + part) * G + hh;
      publish(a.ws_acc + pr * D + d, A);
      if (d == 0) {
        publish(a.ws_ml + pr * 2 + 0, M);
        publish(a.ws_ml + pr * 2 + 1, L);
      }
    }
  }
  if (nparts == 1) return;

  int32_t* counter = a.counters + (size_t)b * n_groups + gg;
  if (!arrive(counter, nparts, &s_last)) return;

  // Rows of partition p for query head qh (of this workgroup's hpw*G):
  // kv head gg*hpw + qh/G, head qh%G; pieces of one head group are not
  // adjacent across kv heads, so piece_rows maps (p, qh) through both.
  __shared__ float s_pm[64][GH];
  __shared__ float s_pl[64][GH];
  const size_t head_rows = (size_t)a.max_parts * G;
  const size_t grp_base = ((size_t)b * Hkv + (size_t)gg * hpw) * head_rows;
  // merge_pieces reads row piece_rows(p) + qh; with qh spanning kv heads the
  // stride between kv heads is head_rows, so merge one kv head at a time.
  for (int x = 0; x < hpw; ++x) {
    const size_t base = grp_base + x * head_rows;
    merge_pieces<DT, D, GH, NT>(
        a, nparts, G, [&](int p) { return base + (size_t)p * G; },
        out_base + (size_t)x * G * D, s_pm, s_pl);
  }
  reset_counter(counter);
}

template <class DT, int D, int BS, int G>
hipError_t launch_partition_t(const DecodeArgs& a, hipStream_t stream) {
  dim3 grid(a.num_seqs * (a.num_kv_heads / a.heads_per_wg), a.max_parts);
  decode_partition_kernel<DT, D, BS, G, kDecodeWaves><<<grid, kDecodeWaves * 64, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_partition(int dtype, int D, int BS, int G, const DecodeArgs& a,
                            hipStream_t s) {
  return dispatch_decode(dtype, D, BS, G, [&](auto dt, auto d, auto bs, auto g) {
    return launch_partition_t<decltype(dt), decltype(d)::value, decltype(bs)::value,
                              decltype(g)::value>(a, s);
  });
}

}  // namespace pa
