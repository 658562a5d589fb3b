// Decode attention, balanced split ("stream-K" style) over ragged batches.
//
// The work of one call is the list of units (sequence b, kv-head group gg,
// logical block j), ordered by b, then gg, then j; a (b, gg) run of units is a
// segment.  A fixed grid sized to fill the GPU takes equal contiguous shares
// of that list: every workgroup streams the same number of KV bytes, whatever
// the mix of lengths, and no workgroup is launched only to find it has nothing
// to do.  A segment cut by a share boundary leaves one partial state per
// piece (at most two per workgroup: its first and its last segment); the last
// workgroup of a segment to arrive merges the pieces with a log-sum-exp
// reduction in the same launch.  Shares are fixed by workgroup index, so the
// merge order, and the result, does not depend on timing.
//
// Per workgroup: hpw consecutive kv heads (their rows are neighbours in every
// token) with all G query heads of each; wave roles, lane layout and the
// per-row online softmax are those of RowAttn.
#include "attn_common.hpp"

#include "decode_launch.hpp"

namespace pa {

template <class DT, int D, int BS, int G, int NW>
__global__ __launch_bounds__(NW * 64) void decode_streamk_kernel(DecodeArgs a) {
  using Sh = DecodeShape<DT, D, BS, G, NW>;
  using Row = RowAttn<DT, D, BS, G, NW>;
  using S = typename DT::storage;
  constexpr int E = Sh::E, RL = Sh::RL, NI = Sh::NI;
  constexpr int GW = Sh::GW, HS = Sh::HS, GH = Sh::GH;
  constexpr int NT = NW * 64;

  const int w = blockIdx.x;
  const int nwg = gridDim.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keep loops scalar
  const int B = a.num_seqs;
  const int Hq = a.num_q_heads;
  const int Hkv = a.num_kv_heads;
  const int hpw = a.heads_per_wg;
  const int n_groups = Hkv / hpw;
  const int nwt = NW / (hpw * HS);
  const int hw = wave % hpw;
  const int hs = (wave / hpw) % HS;
  const int tw = wave / (hpw * HS);
  const int row = lane / RL;
  const int col = lane % RL;
  const int gh = hpw * G;  // query heads of a workgroup

  __shared__ int s_pref[kStreamKMaxSeqs + 1];  // blocks of sequences [0, b)
  __shared__ float s_acc[NW][GW][D];
  __shared__ float s_m[NW][GW];
  __shared__ float s_l[NW][GW];
  __shared__ float s_pm[64][GH];
  __shared__ float s_pl[64][GH];
  __shared__ int s_last;

  // Blocks per sequence and their prefix sums (one wave; an inclusive scan
  // across 64 lanes per step).  A length outside 0..max_blocks*BS counts as
  // no block: that sequence's rows are filled with NaN below.
  if (wave == 0) {
    int run = 0;
    for (int c = 0; c < B; c += 64) {
      const int bb = c + lane;
      int nb = 0;
      if (bb < B) {
        const int cx = a.context_lens[bb];
        if (cx > 0 && cx <= a.max_blocks * BS) nb = (cx + BS - 1) / BS;
      }
      int x = nb;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o);
        if (lane >= o) x += y;
      }
      if (bb < B) s_pref[bb + 1] = run + x;
      run += __shfl(x, 63);
    }
    if (lane == 0) s_pref[0] = 0;
  }
  __syncthreads();

  const int64_t U = (int64_t)n_groups * s_pref[B];
  // Shares go to the first min(grid, U) workgroups, so every share holds at
  // least one unit and the workgroups owning a segment are consecutive.
  const int64_t nsh = U < nwg ? U : nwg;
  auto share_start = [&](int64_t wg) -> int64_t { return wg * U / nsh; };
  // the workgroup whose share holds unit x (largest wg with share_start <= x)
  auto owner = [&](int64_t x) -> int64_t { return ((x + 1) * nsh - 1) / U; };

  // Sequences with no block: zero rows (length 0) or NaN rows (length
  // outside the table), dealt out over the workgroups.
  for (int bb = w; bb < B; bb += nwg) {
    if (s_pref[bb + 1] == s_pref[bb]) {
      const float fill = a.context_lens[bb] == 0 ? 0.0f : __builtin_nanf("");
      const size_t base = (size_t)bb * Hq * D;
      for (int e = tid; e < Hq * D; e += NT) store_out(DT{}, a.out, base + e, fill);
    }
  }

  if (w >= nsh) return;
  const int64_t u0 = share_start(w), u1 = share_start(w + 1);
  const size_t tok_stride = (size_t)Hkv * D;
  const size_t blk_stride = tok_stride * BS;
  const int lane_off = row * Hkv * D + col * E;

  int64_t x = u0;
  while (x < u1) {
    // The segment holding unit x: largest b with n_groups * pref[b] <= x.
    int lo = 0, hi = B;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if ((int64_t)n_groups * s_pref[mid] <= x) lo = mid; else hi = mid;
    }
    const int b = lo;
    const int nb = s_pref[b + 1] - s_pref[b];
    const int64_t first = (int64_t)n_groups * s_pref[b];
    const int gg = (int)((x - first) / nb);
    const int64_t seg_start = first + (int64_t)gg * nb;
    const int64_t seg_end = seg_start + nb;
    const int j_lo = (int)(x - seg_start);
    const int j_hi = (int)((u1 < seg_end ? u1 : seg_end) - seg_start);
    const bool whole = j_lo == 0 && j_hi == nb;
    x = seg_start + j_hi;

    const int g = gg * hpw + hw;
    const int ctx = a.context_lens[b];
    Row st;
    st.load_q(static_cast<const S*>(a.q) + ((size_t)b * Hq + g * G + hs * GW) * D, col);
    st.reset();
    const S* kbase = static_cast<const S*>(a.k_cache) + (size_t)g * D + lane_off;
    const S* vbase = static_cast<const S*>(a.v_cache) + (size_t)g * D + lane_off;
    const int32_t* trow = a.block_tables + (size_t)b * a.max_blocks;
    bool poisoned = false;

    // Table entries in chunks of 64 (lane i holds entry c0 + i), two blocks
    // in flight per wave within a chunk.
    for (int c0 = j_lo; c0 < j_hi; c0 += 64) {
      const int n = min(64, j_hi - c0);
      const int my_blk = lane < n ? trow[c0 + lane] : 0;
      if (__ballot(lane < n && (my_blk < 0 || my_blk >= a.num_blocks)) != 0) {
        poisoned = true;  // same in every wave: nothing of this chunk is read
        continue;
      }
      auto fetch = [&](int jj, uint4 (&kr)[NI], uint4 (&vr)[NI]) {
        const size_t off = (size_t)__builtin_amdgcn_readlane(my_blk, jj) * blk_stride;
        Row::fetch(kbase + off, vbase + off, tok_stride, kr, vr);
      };
      auto consume = [&](int jj, const uint4 (&kr)[NI], const uint4 (&vr)[NI]) {
        const int j = c0 + jj;
        st.consume(j * BS + row, ctx, (j + 1) * BS <= ctx, a.scale_log2, kr, vr);
      };
      uint4 kA[NI], vA[NI], kB[NI], vB[NI];
      int jj = tw;
      if (jj < n) fetch(jj, kA, vA);
      while (jj < n) {
        const int j1 = jj + nwt;
        if (j1 < n) fetch(j1, kB, vB);
        consume(jj, kA, vA);
        if (j1 >= n) break;
        const int j2 = j1 + nwt;
        if (j2 < n) fetch(j2, kA, vA);
        consume(j1, kB, vB);
        jj = j2;
      }
    }
    st.merge_rows();
    st.to_lds(s_acc[wave], s_m[wave], s_l[wave], lane);
    __syncthreads();

    // Waves on one (kv head, head slice) -> this piece's state per element
    // e = (kv head of the group, query head of its group, d).
    const size_t out_base = ((size_t)b * Hq + (size_t)gg * gh) * D;
    const int slot = seg_start <= u0 ? 0 : 1;  // first segment of the share: slot 0
    const size_t piece_row = ((size_t)w * 2 + slot) * gh;
    for (int e = tid; e < gh * D; e += NT) {
      const int hwe = e / (G * D), rem = e % (G * D);
      const int hh = rem / D, d = rem % D;
      const int w0 = hwe + hpw * (hh / GW);
      const int h = hh % GW;
      float M = kNoMax;
      for (int t = 0; t < nwt; ++t) M = fmaxf(M, s_m[w0 + hpw * HS * t][h]);
      float L = 0.0f, A = 0.0f;
      for (int t = 0; t < nwt; ++t) {
        const int wv = w0 + hpw * HS * t;
        const float f = fast_exp2(s_m[wv][h] - M);
        L += s_l[wv][h] * f;
        A += s_acc[wv][h][d] * f;
      }
      if (poisoned) L = __builtin_nanf("");
      if (whole) {
        store_out(DT{}, a.out, out_base + e, A / L);
      } else {
        const size_t r = piece_row + hwe * G + hh;
        publish(a.ws_acc + r * D + d, A);
        if (d == 0) {
          publish(a.ws_ml + r * 2 + 0, M);
          publish(a.ws_ml + r * 2 + 1, L);
        }
      }
    }
    __syncthreads();  // LDS state is reused by the next piece
    if (whole) continue;

    const int64_t w_a = owner(seg_start), w_b = owner(seg_end - 1);
    const int npieces = (int)(w_b - w_a + 1);
    int32_t* counter = a.counters + (size_t)b * n_groups + gg;
    if (arrive(counter, npieces, &s_last)) {
      const bool a_late = share_start(w_a) < seg_start;  // segment began inside w_a's share
      merge_pieces<DT, D, GH, NT>(
          a, npieces, gh,
          [&](int p) -> size_t {
            const int slot_p = (p == 0 && a_late) ? 1 : 0;
            return ((size_t)(w_a + p) * 2 + slot_p) * gh;
          },
          out_base, s_pm, s_pl);
      reset_counter(counter);
    }
  }
}

template <class DT, int D, int BS, int G>
hipError_t launch_streamk_t(const DecodeArgs& a, int num_wg, hipStream_t stream) {
  decode_streamk_kernel<DT, D, BS, G, kDecodeWaves>
      <<<num_wg, kDecodeWaves * 64, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_streamk(int dtype, int D, int BS, int G, const DecodeArgs& a,
                          int num_wg, hipStream_t s) {
  return dispatch_decode(dtype, D, BS, G, [&](auto dt, auto d, auto bs, auto g) {
    return launch_streamk_t<decltype(dt), decltype(d)::value, decltype(bs)::value,
                            decltype(g)::value>(a, num_wg, s);
  });
}

int streamk_wgs_per_cu(int dtype, int D, int BS, int G) {
  int n = 0;
  const hipError_t err = dispatch_decode(dtype, D, BS, G, [&](auto dt, auto d, auto bs, auto g) {
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &n,
        reinterpret_cast<const void*>(
            decode_streamk_kernel<decltype(dt), decltype(d)::value, decltype(bs)::value,
                                  decltype(g)::value, kDecodeWaves>),
        kDecodeWaves * 64, 0);
  });
  return err == hipSuccess ? n : 0;
}

}  // namespace pa
