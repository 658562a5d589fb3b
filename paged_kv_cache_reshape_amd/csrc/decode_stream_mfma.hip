// Decode attention on the balanced schedule (stream_sched.hpp) with the
// matrix-core worker: bfloat16, 4 query heads per kv head.
//
// The schedule is that of decode_stream.hip -- each kv head's block list cut
// into equal ranges, one wave per range, up to four neighbouring kv heads
// per workgroup over one or more consecutive ranges (eight waves at head_dim
// 64, four at 128), split sequences merged by the worker holding their last
// block (stream_merge_last) -- and the fold of a block is that of the
// matrix-core decode (mfma_attn.hpp): the wave stages the block's K and V
// rows of its kv head in its own LDS tile and runs q.k and p.v as 16x16x32
// MFMAs over its G query rows.  With four query heads per kv head the
// vector-ALU worker's multiply-adds and reductions per byte, which grow
// with G, set its pace rather than HBM.
//
// Rows of a block at or past the sequence's length are zeroed in registers
// before staging (the rows exist -- the block is in the pool -- but may hold
// anything, and a zero weight times a NaN value would still be NaN); a block
// whose table entry lies outside the pool is read from block 0, zeroed and
// marks its sequence's rows NaN.  In a decode step the block holding
// position ctx - 1 takes the step's new rows in place of what it read there;
// copy workgroups after the workers store them (step_copy), and nothing in
// the launch reads the stored copy.
#include "mfma_attn.hpp"
#include "stream_sched.hpp"
#include "timeline.hpp"

#include "decode_launch.hpp"

namespace pa {

template <int D, int BS, int G, bool FUSED>
__global__ __launch_bounds__(stream_mfma_waves(D) * 64) void decode_stream_mfma_kernel(DecodeArgs a) {
  constexpr int NW = stream_mfma_waves(D);
  using Sh = TileShape<D, BS, G>;
  using Tile = RowTileAttn<D, BS, G>;
  constexpr int RL = Sh::RL, ROWS = Sh::ROWS, NI = Sh::NI;
  constexpr int KPITCH = Sh::KPITCH, VPITCH = Sh::VPITCH;
  constexpr int KTILE = Sh::KTILE, VTILE = Sh::VTILE;
  constexpr int HT = Sh::HT, DK = Sh::DK, DT = Sh::DT;
  constexpr int NT = NW * 64;
  constexpr int PF = 2;  // blocks in flight per wave
  static_assert(G == 4, "one 16-row tile of query heads, merged in one pass");

  __shared__ int s_cum[kStreamMaxSeqs + 1];
  __shared__ int s_part[NW];
  __shared__ __attribute__((aligned(16))) char s_tile[NW][KTILE + VTILE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int Hkv = a.num_kv_heads, Hq = a.num_q_heads;
  const WaveStamps stamps(blockIdx.x * NW + wave);
  PA_STAMP(stamps, 0);
  const int HW = stream_heads_per_wg(Hkv);
  const int RW = NW / HW;
  const int ngr = Hkv / HW;
  if constexpr (FUSED) {
    if (step_copy_role<BF16, D, BS, NT>(a, ngr * (a.stream_workers / RW))) return;
  }
  const int gg = blockIdx.x % ngr, kwg = blockIdx.x / ngr;
  const int h = gg * HW + wave % HW;
  const int wgs_per_group = a.stream_workers / RW;

  auto empty_rows = [&](int b, int c) {
    if (b % wgs_per_group != kwg) return;
    const size_t base = ((size_t)b * Hq + (size_t)gg * HW * G) * D;
    const float fill = c == 0 ? 0.0f : __builtin_nanf("");
    for (int e = 0; e < HW * G * D; ++e) store_out(BF16{}, a.out, base + e, fill);
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
  const int R = min(a.stream_workers, T);
  const int r = kwg * RW + wave / HW;
  if (r >= R) return;
  StreamRange w;
  if (small)
    stream_range_small(a, sm_start, sm_len, T, R, r, lane, w);
  else
    stream_range(a, s_cum, T, R, r, lane, w);
  PA_STAMP_IDS(stamps);

  const int row = lane / RL, col = lane % RL;
  const int qn = lane & 15, qj = lane >> 4;  // MFMA lane coordinates
  const uint32_t tok_bytes = (uint32_t)Hkv * D * 2;
  const uint32_t blk_bytes = tok_bytes * BS;
  const uint32_t head_off = (uint32_t)h * D * 2 + 16 * col;
  const char* kbase = static_cast<const char*>(a.k_cache);
  const char* vbase = static_cast<const char*>(a.v_cache);
  const uint16_t* qbase = static_cast<const uint16_t*>(a.q) + (size_t)h * G * D;
  const uint16_t* nkbase =
      FUSED ? static_cast<const uint16_t*>(a.new_k) + (size_t)h * D + col * 8 : nullptr;
  const uint16_t* nvbase =
      FUSED ? static_cast<const uint16_t*>(a.new_v) + (size_t)h * D + col * 8 : nullptr;
  const QScale qs(a.scale_log2);

  // Per block: K and V rows (lane (row, col): 16 bytes at d = 8 col of token
  // i ROWS + row), this wave's q rows in the MFMA operand layout (lane
  // (qj, qn): row qn, d = 32 i + 8 qj; rows past G are zero) and, in a
  // decode step, the sequence's new K/V rows.
  struct Slot {
    uint4 k[NI], v[NI], q[HT][DK], nk, nv;
  };
  // A prefetch past the range's end (live false) gets a resource of zero
  // bytes: its loads return zeros and read nothing.
  auto fetch = [&](int i, bool live, Slot& sl) {
    const size_t boff = (size_t)w.entry(i) * blk_bytes;
    const int b = (w.seqblk(i) >> 16) & 0x7FFF;
    const uint32_t nrec = live ? blk_bytes : 0u;
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(kbase + boff), 0, nrec, kBufferRsrcWord3);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(vbase + boff), 0, nrec, kBufferRsrcWord3);
#pragma unroll
    for (int t = 0; t < NI; ++t)
      sl.k[t] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                              rk, head_off + (t * ROWS + row) * tok_bytes, 0,
                                              kLoadStreaming));
#pragma unroll
    for (int t = 0; t < NI; ++t)
      sl.v[t] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                              rv, head_off + (t * ROWS + row) * tok_bytes, 0,
                                              kLoadStreaming));
    const uint16_t* qrow = qbase + (size_t)b * Hq * D;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
      for (int d = 0; d < DK; ++d)
        sl.q[ht][d] = 16 * ht + qn < G
                          ? load_chunk(qrow + (size_t)(16 * ht + qn) * D + 32 * d + 8 * qj)
                          : make_uint4(0, 0, 0, 0);
    if constexpr (FUSED) {
      sl.nk = load_chunk(nkbase + (size_t)b * Hkv * D);
      sl.nv = load_chunk(nvbase + (size_t)b * Hkv * D);
    }
  };

  Tile st;
  int seg_i = 0, seg_j = 0;
  bool poisoned = false;
  // The sequence whose partial state this worker leaves in slot 0, as in the
  // vector-ALU worker; -1 for none.
  int pend0;
  {
    const int v0 = w.seqblk(0);
    const int b0 = (v0 >> 16) & 0x7FFF, j0 = v0 & 0xFFFF;
    const int nb0 = (w.ctx(0) + BS - 1) / BS;
    const bool first_whole = j0 == 0 && nb0 - j0 <= w.n;
    pend0 = first_whole ? -1 : b0;
  }
  const int p0b = max(pend0, 0);
  const SeqPieces sp0(seq_start(p0b), seq_start(p0b + 1) - seq_start(p0b), T, R);
  // The state of the range's first sequence, kept until the range is done
  // (a store in the middle of the stream would hold up later load waits).
  f32x4 first_o[HT][DT];
  float first_m[HT], first_l[HT];

  // Partial state to the workspace: G rows of D floats, then G (max, sum).
  // o's register r of lane (qj, qn) is row 16 ht + 4 qj + r at d = 16 dt + qn.
  auto publish_state = [&](int slot, const f32x4 (&o)[HT][DT], const float (&m)[HT],
                           const float (&l)[HT]) {
    const size_t pr0 = stream_piece_row(h, r, slot, 0, R, G);
    const CoherentRegion racc(a.ws_acc + pr0 * D, G * D * 4);
    const CoherentRegion rml(a.ws_ml + pr0 * 2, G * 2 * 4);
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int gq = 16 * ht + 4 * qj + rr;
        if (gq < G) {
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
            __builtin_amdgcn_raw_buffer_store_b32(ws_encode(o[ht][dt][rr]), racc.r,
                                                  (gq * D + 16 * dt + qn) * 4, 0, kSystemCoherent);
        }
      }
      if (qj == 0 && 16 * ht + qn < G)
        rml.store2u((16 * ht + qn) * 8, ws_encode(m[ht]), ws_encode(l[ht]));
    }
  };

  // End of the sequence's blocks held by this worker.
  auto finish = [&](int b, int j, int nb) {
    float l[HT];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) l[ht] = poisoned ? __builtin_nanf("") : st.row_sum(ht);
    if (seg_j == 0 && j == nb - 1) {
      uint16_t* o = static_cast<uint16_t*>(a.out) + ((size_t)b * Hq + (size_t)h * G) * D;
      st.store_rows([&](int gq, int d, float x) {
        o[(size_t)gq * D + d] = f32_to_bf16_rne(poisoned ? __builtin_nanf("") : x);
      }, lane);
    } else if (seg_i == 0) {
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) {
        first_m[ht] = st.m[ht];
        first_l[ht] = l[ht];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) first_o[ht][dt] = st.o[ht][dt];
      }
    } else {
      // The range's last sequence: the range is done, publish at once.
      publish_state(1, st.o, st.m, l);
    }
  };

  char* kt = s_tile[wave];
  char* vt = kt + KTILE;
  auto consume = [&](int i, Slot& sl) {
    // Everything read back from the lanes (readlane) is read here, with every
    // lane active.
    const int v = w.seqblk(i);
    const int b = (v >> 16) & 0x7FFF, j = v & 0xFFFF;
    const bool bad = v < 0;
    const int ctx = w.ctx(i);
    const int nb = (ctx + BS - 1) / BS;
    const int pos0 = j * BS;
    if (i == 0 || j == 0) {
      st.reset();
      seg_i = i;
      seg_j = j;
      poisoned = false;
#pragma unroll
      for (int ht = 0; ht < HT; ++ht)
#pragma unroll
        for (int d = 0; d < DK; ++d) st.qb[ht][d] = __builtin_bit_cast(bf16x8, qs.apply(sl.q[ht][d]));
    }
    poisoned = poisoned || bad;
    if constexpr (FUSED) {
      if (j == nb - 1) {
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
    // Stage the block in this wave's tile, rows past the length (or every
    // row of a block outside the pool) as zeros.
#pragma unroll
    for (int ii = 0; ii < NI; ++ii) {
      const int tok = ii * ROWS + row;
      const bool keep = !bad && pos0 + tok < ctx;
      *reinterpret_cast<uint4*>(kt + tok * KPITCH + col * 16) = keep ? sl.k[ii] : make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>(vt + tok * VPITCH + col * 16) = keep ? sl.v[ii] : make_uint4(0, 0, 0, 0);
    }
    __builtin_amdgcn_wave_barrier();
    int rowpos[HT];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) rowpos[ht] = !bad && 16 * ht + qn < G ? ctx - 1 : -1;
    st.consume(kt, vt, pos0, rowpos, bad || pos0 + BS > ctx, qs.c, lane);
    __builtin_amdgcn_wave_barrier();
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
  if (pend0 >= 0) publish_state(0, first_o, first_m, first_l);
  // A split sequence is merged in this launch by the wave holding its last
  // piece (or by the merge kernel that follows, with deferred_merge); that
  // piece is always this wave's first sequence, slot 0.
  if (pend0 < 0 || r != sp0.r1 || a.deferred_merge) {
    PA_STAMP(stamps, 3);
    PA_STAMP_VALUE(stamps, 5, 0ull);
    return;
  }
  __builtin_amdgcn_s_waitcnt(0);  // this wave's own published state has landed
  stream_merge_last<BF16, D, G>(a, pend0, h, sp0, R, lane);
  PA_STAMP(stamps, 3);
  PA_STAMP_VALUE(stamps, 5, 1ull + (unsigned long long)(sp0.r1 - sp0.r0));
}

bool stream_mfma_supported(int dtype, int G) { return dtype == PA_DTYPE_BF16 && G == 4; }

hipError_t launch_stream_mfma(int D, int BS, int G, const DecodeArgs& a, hipStream_t s) {
  const int HW = stream_heads_per_wg(a.num_kv_heads);
  const bool fused = a.new_k != nullptr;
  auto go = [&](auto d, auto bs, auto g) -> hipError_t {
    constexpr int Dv = decltype(d)::value, BSv = decltype(bs)::value, Gv = decltype(g)::value;
    constexpr int NW = stream_mfma_waves(Dv);
    const int copy_wgs = step_copy_workgroups(a, Dv, 2, NW * 64);
    const dim3 grid((unsigned)(a.num_kv_heads / HW * (a.stream_workers / (NW / HW)) + copy_wgs));
    if (fused)
      decode_stream_mfma_kernel<Dv, BSv, Gv, true><<<grid, NW * 64, 0, s>>>(a);
    else
      decode_stream_mfma_kernel<Dv, BSv, Gv, false><<<grid, NW * 64, 0, s>>>(a);
    return hipGetLastError();
  };
  if (G != 4) return hipErrorInvalidValue;
  auto by_bs = [&](auto d) -> hipError_t {
    return BS == 16 ? go(d, IntC<16>{}, IntC<4>{}) : go(d, IntC<32>{}, IntC<4>{});
  };
  return D == 64 ? by_bs(IntC<64>{}) : by_bs(IntC<128>{});
}

}  // namespace pa

PA_TIMELINE_READER(pa_debug_timeline_mfma)
