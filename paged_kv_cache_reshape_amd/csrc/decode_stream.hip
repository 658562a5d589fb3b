// Decode attention on the balanced schedule (stream_sched.hpp), vector-ALU
// worker: every wave is an independent worker over an equal range of one kv
// head's block list, holding the G query heads of that kv head for one
// sequence at a time (the per-row online softmax of RowAttn).  A workgroup
// is kStreamWaves workers of the same kv head over consecutive ranges; after
// the shared prefix sum there is no workgroup barrier, and no cross-wave
// combine: a wave finishes each sequence it holds on its own.
//
// Per block the wave loads the K and V rows of its kv head (full-row 16-byte
// loads, two blocks in flight), the query rows of the block's sequence (a
// 512-byte read that hits the L2 after the sequence's first block) and, in a
// decode step, the step's new K/V rows.  In a decode step the block holding
// position ctx - 1 takes the new rows in place of what it read there; copy
// workgroups after the workers store them (step_copy): nothing in the launch
// reads the stored copy, so the result is the write followed by the read,
// bit for bit.
#include "stream_sched.hpp"
#include "timeline.hpp"

#include "decode_launch.hpp"

namespace pa {

// 16-byte chunk of E output values: bf16 rounded to nearest even, or f32.
__device__ __forceinline__ uint4 out_chunk(BF16, const float* x) {
  uint32_t w[4];
#pragma unroll
  for (int k = 0; k < 4; ++k)
    w[k] = (uint32_t)f32_to_bf16_rne(x[2 * k]) | ((uint32_t)f32_to_bf16_rne(x[2 * k + 1]) << 16);
  return make_uint4(w[0], w[1], w[2], w[3]);
}
__device__ __forceinline__ uint4 out_chunk(F32, const float* x) {
  return make_uint4(__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]),
                    __float_as_uint(x[3]));
}

template <class DT, int D, int BS, int G, bool FUSED>
__global__ __launch_bounds__(kStreamWaves * 64) void decode_stream_kernel(DecodeArgs a) {
  using Sh = DecodeShape<DT, D, BS, G, 1>;
  using Row = RowAttn<DT, D, BS, G, 1>;
  using S = typename DT::storage;
  constexpr int E = Sh::E, RL = Sh::RL, ROWS = Sh::ROWS, NI = Sh::NI;
  constexpr int NT = kStreamWaves * 64;
  // Two blocks in flight; one where a block's rows already take 64 registers
  // for K and V (float32 at head_dim 128 with 32-token blocks).
  constexpr int PF = NI <= 8 ? 2 : 1;
  static_assert(G <= 8, "one wave holds every query head of its kv head");

  __shared__ int s_cum[kStreamMaxSeqs + 1];
  __shared__ int s_part[kStreamWaves];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int Hkv = a.num_kv_heads, Hq = a.num_q_heads;
  const WaveStamps stamps(blockIdx.x * kStreamWaves + wave);
  PA_STAMP(stamps, 0);
  if constexpr (FUSED) {
    const int hw = stream_heads_per_wg(Hkv);
    if (step_copy_role<DT, D, BS, NT>(a, Hkv / hw * (a.stream_workers / (kStreamWaves / hw))))
      return;
  }
  // The workgroup's waves take HW neighbouring kv heads (one each) of RW
  // consecutive ranges: their loads then cover HW * D * elt contiguous bytes
  // of each token row, which measured far steadier per-wave rates than waves
  // of one head over four ranges (MI355X, Qwen3-shaped batch: streaming
  // times spread 19-29 us across waves with one head per workgroup).
  const int HW = stream_heads_per_wg(Hkv);
  const int RW = kStreamWaves / HW;
  const int ngr = Hkv / HW;
  const int gg = blockIdx.x % ngr, kwg = blockIdx.x / ngr;
  const int h = gg * HW + wave % HW;
  const int wgs_per_group = a.stream_workers / RW;

  // Empty sequences give zero rows, lengths past the table NaN rows; each is
  // written for this workgroup's kv heads by one workgroup of the group.
  auto empty_rows = [&](int b, int c) {
    if (b % wgs_per_group != kwg) return;
    const size_t base = ((size_t)b * Hq + (size_t)gg * HW * G) * D;
    const float fill = c == 0 ? 0.0f : __builtin_nanf("");
    for (int e = 0; e < HW * G * D; ++e) store_out(DT{}, a.out, base + e, fill);
  };
  // Up to 64 sequences: the set-up in each wave's registers; else through LDS.
  const bool small = a.num_seqs <= kStreamSmallSeqs;
  int sm_start = 0, sm_len = 0;
  const int T = small ? stream_prefix_small(a, BS, lane, wave == 0, sm_start, sm_len, empty_rows)
                      : stream_prefix<NT>(a, BS, s_cum, s_part, empty_rows);
  // First block of sequence b in the kv head's list (b <= B, wave-uniform).
  auto seq_start = [&](int b) {
    return small ? small_seq_start(sm_start, b, a.num_seqs, T) : s_cum[b];
  };

  PA_STAMP(stamps, 6);
  // With fewer blocks than workers, the first T workers take one block each
  // and the rest none: every worker in [0, R) then holds a block, which the
  // piece count of a merge relies on.
  const int R = min(a.stream_workers, T);
  const int r = kwg * RW + wave / HW;
  if (r >= R) return;
  StreamRange w;
  if (small)
    stream_range_small(a, sm_start, sm_len, T, R, r, lane, w);
  else
    stream_range(a, s_cum, T, R, r, lane, w);
  PA_STAMP(stamps, 7);
  PA_STAMP_IDS(stamps);

  const int row = lane / RL, col = lane % RL;
  const size_t tok_stride = (size_t)Hkv * D;
  const size_t blk_stride = tok_stride * BS;
  const uint32_t tok_bytes = (uint32_t)(tok_stride * sizeof(S));
  const uint32_t blk_bytes = tok_bytes * BS;
  const uint32_t lane_bytes = (uint32_t)(((size_t)row * tok_stride + (size_t)h * D + col * E) * sizeof(S));
  const char* kbase = static_cast<const char*>(a.k_cache);
  const char* vbase = static_cast<const char*>(a.v_cache);
  const S* qbase = static_cast<const S*>(a.q) + (size_t)h * G * D + col * E;
  const S* nkbase = FUSED ? static_cast<const S*>(a.new_k) + (size_t)h * D + col * E : nullptr;
  const S* nvbase = FUSED ? static_cast<const S*>(a.new_v) + (size_t)h * D + col * E : nullptr;

  struct Slot {
    uint4 k[NI], v[NI], q[G], nk, nv;
  };
  // Block i's rows through buffer loads over that block (16 bytes a lane at
  // d = E col of token t ROWS + row).  The resource covers the rows below the
  // sequence's length only: rows past it in the last block read nothing (they
  // return zeros, and are masked anyway).  A prefetch past the range's end
  // (live false) gets a resource of zero bytes: its loads return zeros and
  // read nothing, where re-reading the last block would cost a block of HBM
  // traffic per wave.
  auto fetch = [&](int i, bool live, Slot& sl) {
    const size_t off = (size_t)w.entry(i) * blk_stride * sizeof(S);
    const int b = (w.seqblk(i) >> 16) & 0x7FFF;
    const int rows = min(BS, w.ctx(i) - (w.seqblk(i) & 0xFFFF) * BS);  // >= 1
    const uint32_t n = live ? (uint32_t)rows * tok_bytes : 0u;
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(kbase + off), 0, n, kBufferWord3);
    const __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(vbase + off), 0, n, kBufferWord3);
#pragma unroll
    for (int t = 0; t < NI; ++t)
      sl.k[t] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                              rk, lane_bytes + t * ROWS * tok_bytes, 0, kLoadNT));
#pragma unroll
    for (int t = 0; t < NI; ++t)
      sl.v[t] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                              rv, lane_bytes + t * ROWS * tok_bytes, 0, kLoadNT));
#pragma unroll
    for (int gh = 0; gh < G; ++gh) sl.q[gh] = load_chunk(qbase + ((size_t)b * Hq + gh) * D);
    if constexpr (FUSED) {
      sl.nk = load_chunk(nkbase + (size_t)b * tok_stride);
      sl.nv = load_chunk(nvbase + (size_t)b * tok_stride);
    }
  };

  Row st;
  int seg_i = 0, seg_j = 0;
  bool poisoned = false;
  // The sequence whose partial state this worker leaves in slot 0 (its range
  // starts inside it, or it continues past the range's end); -1 for none.
  // Wave-uniform, known from the range's first block.  (The range's last
  // sequence, when it starts inside the range and continues past its end,
  // leaves slot 1, published as soon as it is reached.)
  int pend0;
  {
    const int v0 = w.seqblk(0);
    const int b0 = (v0 >> 16) & 0x7FFF, j0 = v0 & 0xFFFF;
    const int nb0 = (w.ctx(0) + BS - 1) / BS;
    const bool first_whole = j0 == 0 && nb0 - j0 <= w.n;
    pend0 = first_whole ? -1 : b0;
  }
  // Where its pieces lie, worked out now rather than after the stream, when
  // the merge is on the launch's critical path.
  const int p0b = max(pend0, 0);
  const SeqPieces sp0(seq_start(p0b), seq_start(p0b + 1) - seq_start(p0b), T, R);
  // The partial state of the range's first sequence, kept in registers until
  // the range is done: a store issued in the middle of the stream would hold
  // up the waits on every load issued after it (one in-order counter covers
  // loads and stores), and a system-scope store takes a memory round trip.
  float first_m[G], first_l[G], first_acc[G][E];

  // Partial state of (this worker, slot) to the workspace, for the merge:
  // the G rows of a piece are contiguous, G * D floats of output, then G
  // (max, sum) pairs; a lane of row group `row` writes its E values of the
  // query heads gh with gh % ROWS == row.
  auto publish_state = [&](int slot, const float (&m)[G], const float (&l)[G],
                           const float (&acc)[G][E]) {
    const size_t pr0 = stream_piece_row(h, r, slot, 0, R, G);
    const CoherentRegion racc(a.ws_acc + pr0 * D, G * D * 4);
    const CoherentRegion rml(a.ws_ml + pr0 * 2, G * 2 * 4);
#pragma unroll
    for (int gh = 0; gh < G; ++gh) {
      if (gh % ROWS == row) {
        const uint32_t off = (gh * D + col * E) * 4;
#pragma unroll
        for (int e = 0; e < E; e += 4) {
          const uint32_t wv[4] = {ws_encode(acc[gh][e]), ws_encode(acc[gh][e + 1]),
                                  ws_encode(acc[gh][e + 2]), ws_encode(acc[gh][e + 3])};
          racc.store4u(off + 4 * e, wv);
        }
        if (col == 0) rml.store2u(gh * 8, ws_encode(m[gh]), ws_encode(l[gh]));
      }
    }
  };

  // End of the sequence's blocks held by this worker: the output rows when
  // the worker held all of them, else the partial state for the merge (a
  // NaN sum when a block of it lay outside the pool).
  auto finish = [&](int b, int j, int nb) {
    st.merge_rows();
    if (seg_j == 0 && j == nb - 1) {
#pragma unroll
      for (int gh = 0; gh < G; ++gh) {
        if (gh % ROWS == row) {
          float x[E];
#pragma unroll
          for (int e = 0; e < E; ++e) x[e] = poisoned ? __builtin_nanf("") : st.acc[gh][e] / st.l[gh];
          S* o = static_cast<S*>(a.out) + ((size_t)b * Hq + (size_t)h * G + gh) * D + col * E;
          store_chunk(o, out_chunk(DT{}, x));
        }
      }
    } else {
      const int slot = seg_i > 0 ? 1 : 0;
      float l[G];
#pragma unroll
      for (int gh = 0; gh < G; ++gh) l[gh] = poisoned ? __builtin_nanf("") : st.l[gh];
      if (slot == 0) {
#pragma unroll
        for (int gh = 0; gh < G; ++gh) {
          first_m[gh] = st.m[gh];
          first_l[gh] = l[gh];
#pragma unroll
          for (int e = 0; e < E; ++e) first_acc[gh][e] = st.acc[gh][e];
        }
      } else {
        // The range's last sequence: the range is done, publish at once.
        publish_state(1, st.m, l, st.acc);
      }

    }
  };

  auto consume = [&](int i, Slot& sl) {
    // Everything read back from the lanes (readlane) is read here, with every
    // lane active: a value selected per lane inside a divergent branch is not
    // defined in the inactive lanes readlane would read.
    const int v = w.seqblk(i);
    const int b = (v >> 16) & 0x7FFF, j = v & 0xFFFF;
    const bool bad = v < 0;
    const int ctx = w.ctx(i);
    const int nb = (ctx + BS - 1) / BS;
    if (i == 0 || j == 0) {
      st.reset();
      seg_i = i;
      seg_j = j;
      poisoned = false;
    }
    poisoned = poisoned || bad;
    if constexpr (FUSED) {
      if (j == nb - 1) {
        // Position ctx - 1 (token t of this block) holds the step's token.
        const int t = (ctx - 1) % BS;
        const int li = t / ROWS, lr = t % ROWS;
#pragma unroll
        for (int ii = 0; ii < NI; ++ii) {
          if (ii == li && row == lr) {
            sl.k[ii] = sl.nk;
            sl.v[ii] = sl.nv;
          }
        }
      }
    }
#pragma unroll
    for (int gh = 0; gh < G; ++gh) st.qv[gh] = sl.q[gh];
    st.consume(j * BS + row, ctx, !bad, a.scale_log2, sl.k, sl.v);
    if (i == w.n - 1 || j == nb - 1) finish(b, j, nb);
  };

  Slot sl[PF];
  const auto clampi = [&](int i) { return i < w.n ? i : w.n - 1; };
#pragma unroll
  for (int p = 0; p < PF - 1; ++p) {
    fetch(clampi(p), p < w.n, sl[p]);
    __builtin_amdgcn_sched_barrier(0);
  }
  PA_STAMP(stamps, 1);
  for (int i0 = 0; i0 < w.n; i0 += PF) {
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      const int nx = i0 + u + PF - 1;
      fetch(clampi(nx), nx < w.n, sl[(u + PF - 1) % PF]);
      __builtin_amdgcn_sched_barrier(0);
      if (i0 + u < w.n) consume(i0 + u, sl[u]);
    }
  }

  PA_STAMP(stamps, 2);
  if (pend0 >= 0) publish_state(0, first_m, first_l, first_acc);
  // A split sequence is merged in this launch by the wave holding its last
  // piece (or by the merge kernel that follows, with deferred_merge); that
  // piece is always this wave's first sequence, slot 0.
  if (pend0 < 0 || r != sp0.r1 || a.deferred_merge) {
    PA_STAMP(stamps, 3);
    PA_STAMP_VALUE(stamps, 5, 0ull);
    return;
  }
  __builtin_amdgcn_s_waitcnt(0);  // this wave's own published state has landed
  stream_merge_last<DT, D, G>(a, pend0, h, sp0, R, lane);
  PA_STAMP(stamps, 3);
  PA_STAMP_VALUE(stamps, 5, 1ull + (unsigned long long)(sp0.r1 - sp0.r0));
}

// The merges of split sequences as a kernel of their own, launched right
// after the stream kernel: one wave per (sequence, kv head), the prefix sum
// recomputed by each workgroup.  The stream kernel's published states are
// complete and visible once it has ended.
template <class DT, int D, int G>
__global__ __launch_bounds__(kStreamWaves * 64) void stream_merge_kernel(DecodeArgs a, int bs) {
  __shared__ int s_cum[kStreamMaxSeqs + 1];
  __shared__ int s_part[kStreamWaves];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int T = stream_prefix<kStreamWaves * 64>(a, bs, s_cum, s_part, [](int, int) {});
  const int R = min(a.stream_workers, T);
  const int item = blockIdx.x * kStreamWaves + wave;
  const int Hkv = a.num_kv_heads;
  if (item >= a.num_seqs * Hkv) return;
  const int b = item / Hkv, h = item % Hkv;
  const int cb = s_cum[b], nb = s_cum[b + 1] - cb;
  if (nb == 0) return;
  const SeqPieces sp(cb, nb, T, R);
  if (sp.count() > 1) stream_merge<DT, D, G>(a, b, h, sp, R, lane);
}

bool stream_supported(int G) { return G == 1 || G == 2 || G == 4; }

hipError_t launch_stream_merge(int dtype, int D, int BS, int G, const DecodeArgs& a,
                               hipStream_t s) {
  const dim3 grid((unsigned)((a.num_seqs * a.num_kv_heads + kStreamWaves - 1) / kStreamWaves));
  auto go = [&](auto dt, auto d, auto g) -> hipError_t {
    stream_merge_kernel<decltype(dt), decltype(d)::value, decltype(g)::value>
        <<<grid, kStreamWaves * 64, 0, s>>>(a, BS);
    return hipGetLastError();
  };
  auto by_g = [&](auto dt, auto d) -> hipError_t {
    switch (G) {
      case 1: return go(dt, d, IntC<1>{});
      case 2: return go(dt, d, IntC<2>{});
      case 4: return go(dt, d, IntC<4>{});
    }
    return hipErrorInvalidValue;
  };
  auto by_d = [&](auto dt) -> hipError_t {
    return D == 64 ? by_g(dt, IntC<64>{}) : by_g(dt, IntC<128>{});
  };
  return dtype == PA_DTYPE_BF16 ? by_d(BF16{}) : by_d(F32{});
}

hipError_t launch_stream(int dtype, int D, int BS, int G, const DecodeArgs& a, hipStream_t s) {
  const int HW = stream_heads_per_wg(a.num_kv_heads);
  const bool fused = a.new_k != nullptr;
  auto go = [&](auto dt, auto d, auto bs, auto g) -> hipError_t {
    using DT = decltype(dt);
    constexpr int Dv = decltype(d)::value, BSv = decltype(bs)::value, Gv = decltype(g)::value;
    const int copy_wgs =
        step_copy_workgroups(a, Dv, sizeof(typename DT::storage), kStreamWaves * 64);
    const dim3 grid(
        (unsigned)(a.num_kv_heads / HW * (a.stream_workers / (kStreamWaves / HW)) + copy_wgs));
    if (fused)
      decode_stream_kernel<DT, Dv, BSv, Gv, true><<<grid, kStreamWaves * 64, 0, s>>>(a);
    else
      decode_stream_kernel<DT, Dv, BSv, Gv, false><<<grid, kStreamWaves * 64, 0, s>>>(a);
    return hipGetLastError();
  };
  auto by_g = [&](auto dt, auto d, auto bs) -> hipError_t {
    switch (G) {
      case 1: return go(dt, d, bs, IntC<1>{});
      case 2: return go(dt, d, bs, IntC<2>{});
      case 4: return go(dt, d, bs, IntC<4>{});
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

}  // namespace pa


PA_TIMELINE_READER(pa_debug_timeline)
