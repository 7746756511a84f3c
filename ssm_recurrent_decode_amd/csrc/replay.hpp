// ReplaySSM window kernel (append-decode and T-draft verify) and its launcher,
// shared by the translation units that instantiate it.
//
// Method: "ReplaySSM: Cache SSM Inputs, Not State" -- method (core idea,
// output-only decode, rollback as a pointer move), algorithms (Mamba-2 standard
// decode; speculative decoding with the early-flush rule) and kernel design
// (shared inner products, ring indexed in-kernel).
#pragma once

#include "common.hpp"

namespace rssm {

// ======================================================= ReplaySSM
// Draft windows from this size up combine on the matrix cores (measured against
// the vector-ALU dot products, interleaved on the same buffers at B = 512: T = 3
// -0.8 %, T = 4 -2.2 %, and at T = 5, 6 the vector path also costs a wave per
// SIMD in registers; T = 2 was even before the state moved as whole lines and
// -5.8 % after; a one-token call on the matrix cores, 15 of 16 columns unused:
// +3.3 %).
constexpr int kMfmaCombineMinT = 2;

struct ReplayParams {
  float* state0;
  uint16_t* ring_v;
  uint16_t* ring_k;
  float* meta;         // [B, H, meta_words(L)] per-head ring records
  int32_t* err;
  const uint16_t* v;   // [B, T, H, D]
  const uint16_t* k;   // [B, T, G, N]
  const uint16_t* q;   // [B, T, G, N]
  const float* dt;     // [B, T, H]
  const float* dt_bias;
  const float* A;
  float* y;            // [B, T, H, D]
  int32_t* flushed;
  const int32_t* mask;  // explicit flush only
  const int32_t* accepted;  // commit-and-verify: the previous window's accepted drafts, or null
  const int32_t* slots;  // pool row per batch entry, or null
  int rows;
  // fused front-end (append only): depthwise causal conv1d (width 4) + SiLU over
  // the layer's xBC channels [x (H*D) | B (G*N) | C (G*N)] produce v, k, q
  const uint16_t* conv_in;   // bf16 [rows, C, 3] conv state read
  uint16_t* conv_out;        // bf16 [rows, C, 3] conv state written (not conv_in)
  const uint16_t* xbc;       // bf16 [B, C] conv inputs of this token
  const uint16_t* conv_w;    // bf16 [C, 4] taps (the last multiplies the token)
  int y_bf16;                // outputs stored as bf16
  int H, G, L;
};

// fp64 -> bf16 bits, round to nearest even, in one rounding: the value is first
// cut to fp32 toward zero with a sticky last bit (round to odd, 16 spare bits),
// then rounded to bf16 -- the same as rounding the fp64 value directly.
__device__ __forceinline__ uint32_t f64_to_bf16_rne(double x) {
  const float t = __double2float_rz(x);
  uint32_t u = __float_as_uint(t);
  if ((double)t != x) u |= 1u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// SiLU of one channel's 4-tap conv sum, rounded to bf16 exactly as the float64
// value rounds (nearest, ties to even).  fp32 first: the products of bf16 values
// are exact in fp32, the three additions err by at most 3 u S (S = sum of
// |products|, u = 2^-24) and SiLU's slope is below 1.1, while expf (within one
// ulp), the addition and the division add at most 4 u |s|; so a value farther
// than 8 u |s| + 4 u S from the midpoint between its two bf16 neighbours rounds
// as the exact one does.  The few that are not (about 1 in 2 * 10^3; also every
// |z| >= 64) take the float64 route, where the sum of the exact products is
// exact and SiLU is evaluated in float64 before one rounding.
__device__ __forceinline__ uint32_t conv_silu_bf16(const uint32_t* w, const uint32_t* x) {
  float p[4], S = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    p[k] = bf16_to_f32(w[k]) * bf16_to_f32(x[k]);
    S += fabsf(p[k]);
  }
  const float z = ((p[0] + p[1]) + p[2]) + p[3];  // oldest tap first
  const float sf = z / (1.f + expf(-z));
  const float mid = __uint_as_float((__float_as_uint(sf) & 0xFFFF0000u) | 0x8000u);
  const float err = 0x1p-21f * fabsf(sf) + 0x1p-22f * S + 0x1p-126f;
  if (fabsf(sf - mid) > err && fabsf(z) < 64.f) return bf16_rne(sf);
  double zd = (double)bf16_to_f32(w[0]) * (double)bf16_to_f32(x[0]);
#pragma unroll
  for (int k = 1; k < 4; ++k) zd = zd + (double)bf16_to_f32(w[k]) * (double)bf16_to_f32(x[k]);
  return f64_to_bf16_rne(zd / (1.0 + exp(-zd)));
}

// One kernel for both decode modes, one work-group of four waves per (request,
// head).
//  APPEND (T == 1): append the token; it is entry c of E = c + 1; flush all E
//    entries when E == L (flush-when-full).  count <- E or 0.
//  VERIFY (T drafts): drafts are entries c .. c+T-1; draft s reads p_s = c+s+1
//    entries; if c + 2T > L fold the c committed entries only.  pending <- T.
//
// Issue order: this head's ring record (pointer word and step sizes), the
// queries, drafts and new entries, then the checkpoint (line arrangement), then -- once the
// pointer word is in -- the ring keys and values of the c committed entries only
// (on average half the ring).  Loads complete in issue order, so the weights
// (wave 0) go ahead while the checkpoint streams in; the inner products k . q,
// the output combine and the fold follow it.  Ring values arrive 16 bytes per
// lane and are kept in LDS together with the new entries' values, so the
// combine and the fold read every value from one array by physical slot; the
// pointers decide which logical entry a slot holds (j = slot - head mod L).
// Weights are computed in logical order and stored by physical slot.  The new
// entries and the record are written by the last stores of the kernel.  LCAP
// (16 or 32) bounds L and sizes the arrays.
//  CONV (APPEND only): v, k, q are not inputs but the SiLU outputs of the causal
//    conv1d over this head's x channels and its group's B and C channels,
//    rounded to bf16 (the precision of the ring); the conv states of the x
//    channels are written by their head, those of B and C by the group's heads
//    in equal shares, into a second buffer (the group's other heads still read
//    the first).
// Waves per SIMD the fused front-end is held to at d = 64: with the ring loads
// issued before the conv, the conv's operands and the ring registers are live
// together, and left alone the compiler takes 108 registers (four waves per
// SIMD, +6 % per launch); bounded to five it fits in 96 without spilling and
// runs 1 % faster than the conv before the ring loads.  The append-decode at
// d = 64, n = 128 with a ring of up to 32 entries is held to five as well: left
// alone they took 100 vector and 4 accumulator registers (four waves per SIMD),
// and bounded they fit in 96 without spilling and run 7 % faster (append-decode
// at L = 32, 32 and 128 heads, interleaved; at L = 16 the same bound changed
// nothing).  At d = 64, n = 64 (16 KB of checkpoint per work-group) and L <= 16,
// seven waves per SIMD (67 registers, from 72 + 4 accumulator registers at six):
// append -1.0 %, verify -1.2 % per launch, interleaved; eight spilled in the
// verify.  Other instances: no bound.
template <int D, int N, bool APPEND, bool CONV, int LCAP>
constexpr int window_waves_per_simd() {
  return ((CONV && D == 64 && N == 128 && LCAP == 16) || (APPEND && !CONV && D == 64 && N == 128 && LCAP == 32))
             ? 5
             : ((D == 64 && N == 64 && LCAP == 16) ? 7 : 1);
}

template <int D, int N, int T, bool APPEND, int LCAP, bool CONV = false>
__global__ __launch_bounds__(kBlock, (window_waves_per_simd<D, N, APPEND, CONV, LCAP>())) void replay_window_kernel(ReplayParams p) {
  static_assert(N == 64 || N == 128 || N == 256, "keys and queries: 16 lanes of n / 16 values");
  static_assert(LCAP == 16 || LCAP == 32, "ring capacity bound");
  static_assert(!CONV || (APPEND && T == 1), "the fused front-end is one token");
  constexpr int NCONV = D + 2 * N;  // channels of one head: its x, the group's B and C
  // conv channels per thread: two, or four where two would need more threads
  // than the work-group has (n = 256)
  constexpr int CPT = NCONV / 2 <= kBlock ? 2 : 4;
  constexpr int NCQ = NCONV / CPT;   // threads of the conv
  static_assert(!CONV || NCQ <= kBlock, "one pass of the conv");
  constexpr int NCT = N / 16;
  constexpr int RT = D / (16 * kWavesPerBlock);
  constexpr int VJ = LCAP / 4;         // physical slots per lane in the combine and fold
  constexpr int PASSES = LCAP / 16;    // inner-product passes of 16 slots
  constexpr int NEWV = T * D / 8;      // 16-byte chunks of the head's new v
  constexpr int NEWK = T * N / 8;      // ... of the group's new k
  constexpr int NCH = NEWV + NEWK;
  constexpr int NCP = (NCH + kBlock - 1) / kBlock;
  constexpr int RVC = LCAP * D / 8;    // 16-byte chunks of the head's ring values
  constexpr int RVP = (RVC + kBlock - 1) / kBlock;
  using KL = KeyLanes<N>;           // a key or query over 16 lanes, KQC chunks of KQW values each
  using KC = typename KL::Chunk;
  constexpr int KQC = KL::C, KQW = KL::W, KPL = N / 16;
  __shared__ float s_w[T][LCAP];       // w_{j,s} by physical slot, zero where not read
  __shared__ float s_M[T][LCAP];       // k . q_s by physical slot
  __shared__ float s_abar[T];
  __shared__ float s_fw[LCAP];         // fold weights by physical slot
  __shared__ float s_fabar;
  __shared__ float s_dtn[T];  // the new entries' step sizes
  __shared__ __attribute__((aligned(16))) float s_y[T * D];  // outputs, stored whole lines at the end
  __shared__ __attribute__((aligned(16))) uint16_t s_qk[2 * T * N];  // the drafts' q, then their k
  __shared__ __attribute__((aligned(16))) uint16_t s_k[LCAP * N];  // keys to fold by slot
  __shared__ __attribute__((aligned(16))) uint16_t s_v[LCAP * D];  // values by slot
  __shared__ __attribute__((aligned(16))) uint16_t s_conv[CONV ? NCONV : 8];  // v | k | q

  const int H = p.H, G = p.G, L = p.L;
  const int wg = xcd_remap<(APPEND ? kXcdChunkAppend : kXcdChunk)>(blockIdx.x, gridDim.x);
  const int b = wg / H, h = wg - b * H, hpg = H / G, g = h / hpg;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, cq = lane >> 4, sub = lane & 15;
  const int rb = pool_row(p.slots, p.rows, b, p.err, tid == 0 && h == 0);  // request's row
  if (rb < 0) return;                 // padding or outside the pool: whole work-group
  const size_t bh = (size_t)rb * H + h;  // per-(row, head) checkpoint, ring and record

  // ---- 1. this head's ring record (pointer word, step sizes) and every small operand
  const int MS = meta_words(L);
  float* rec = p.meta + bh * MS;  // this head's ring record
  // (both read per lane, so that the checkpoint loads are issued before they arrive)
  const int z0 = opaque_zero();
  const unsigned long long word = *reinterpret_cast<const unsigned long long*>(rec + kMetaPtr + z0);
  const int acc_prev = (!APPEND && p.accepted != nullptr) ? p.accepted[b + z0] : 0;
  // The token's query and key: each lane keeps the 16-lane slices it needs in
  // registers (qm, kin).  Several drafts would hold 2T such slices per lane
  // across the checkpoint load (a wave per SIMD fewer), so from T = 2 they are
  // loaded one 16-byte chunk per thread and staged into LDS once the checkpoint
  // loads are issued; the inner products read them from there (measured on the
  // speculative workload, B = 512, T = 4: -5 % per round; at T = 1 the extra
  // barrier costs 1 %).
  constexpr bool kQkLds = T > 1;
  constexpr int QKC = 2 * T * N / 8;
  constexpr int QKP = kQkLds ? (QKC + kBlock - 1) / kBlock : 1;
  constexpr int TQ = kQkLds ? 1 : T;  // register slices
  uint4 qkc[QKP];
  KC qm[TQ][KQC], kin[TQ][KQC];
  uint4 newc[NCP];  // chunks of the new entries: the head's v, then the group's k
  // conv operands of the channels this thread computes (CONV only), per pair of
  // channels: state 2 x 3 bf16 (one 12-byte load), the token 2 bf16, the taps
  // 2 x 4 bf16.  Two channels per thread (160 threads at d = 64, n = 128)
  // instead of four over 80: every state load and store instruction covers its
  // bytes whole, and each thread's SiLU chain is half as long (-2.3 % per
  // launch, interleaved; bit-identical)
  constexpr int CPR = CPT / 2;  // pairs of channels per thread
  int cch = 0;
  v3u cst[CPR];
  uint32_t cxv[CPR];
  uint4 cwv[CPR];
  if constexpr (!CONV) {
    if constexpr (kQkLds) {
#pragma unroll
      for (int i = 0; i < QKP; ++i) {
        const int t = min(tid + i * kBlock, QKC - 1);
        const int v = t / (N / 8), o = (t % (N / 8)) * 8;  // vector (q_0..q_{T-1}, k_0..k_{T-1}), column
        qkc[i] = ld_u4((v < T ? p.q : p.k) + (((size_t)b * T + (v < T ? v : v - T)) * G + g) * N + o);
      }
    } else {
#pragma unroll
      for (int ch = 0; ch < KQC; ++ch) {
        qm[0][ch] = *reinterpret_cast<const KC*>(p.q + ((size_t)b * G + g) * N + sub * KPL + ch * KQW);
        kin[0][ch] = *reinterpret_cast<const KC*>(p.k + ((size_t)b * G + g) * N + sub * KPL + ch * KQW);
      }
    }
#pragma unroll
    for (int i = 0; i < NCP; ++i) {
      const int t = min(tid + i * kBlock, NCH - 1);
      const uint16_t* src;
      if (t < NEWV) {
        src = p.v + (((size_t)b * T + t / (D / 8)) * H + h) * D + (t % (D / 8)) * 8;
      } else {
        const int tk = t - NEWV;
        src = p.k + (((size_t)b * T + tk / (N / 8)) * G + g) * N + (tk % (N / 8)) * 8;
      }
      newc[i] = ld_u4(src);
    }
  } else {
    if (tid < NCQ) {
      const int C = H * D + 2 * G * N;
      const int lc = CPT * tid;  // first local channel: x | B | C (never straddling two)
      cch = lc < D ? h * D + lc : (lc < D + N ? H * D + g * N + (lc - D) : H * D + G * N + g * N + (lc - D - N));
#pragma unroll
      for (int i = 0; i < CPR; ++i) {
        cst[i] = __builtin_nontemporal_load(reinterpret_cast<const v3u*>(p.conv_in + ((size_t)rb * C + cch + 2 * i) * 3));
        cxv[i] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p.xbc + (size_t)b * C + cch + 2 * i));
        cwv[i] = *reinterpret_cast<const uint4*>(p.conv_w + (size_t)(cch + 2 * i) * 4);
      }
    }
  }
  float rec_l = 0.f, dt_draft = 0.f, dt_bias = 0.f, A_h = 0.f;
  if (wave == 0) {  // the whole record (step sizes of every slot), the drafts' raw dt
    rec_l = rec[min(lane, MS - 1)];
    dt_draft = p.dt[((size_t)b * T + min(lane, T - 1)) * H + h];
    dt_bias = p.dt_bias[h];
    A_h = p.A[h];
  }

  // ---- 2. the checkpoint (the scheduler may not hoist it above the rest), in the
  //      line arrangement: each pair of column tiles is settled into the tile
  //      layout where the combine first uses it
  __builtin_amdgcn_sched_barrier(0);
  float4 st[RT][NCT];
  load_state_lines<N, RT, NCT>(st, p.state0 + bh * D * N, wave, r, cq);
  if constexpr (!CONV && kQkLds) {
#pragma unroll
    for (int i = 0; i < QKP; ++i) {
      const int t = tid + i * kBlock;
      if (t < QKC) *reinterpret_cast<uint4*>(&s_qk[t * 8]) = qkc[i];
    }
  }

  // ---- 3. ring pointers (uniform per request), clamped into range
  const RingPtr rp = unpack_ptr(word);
  int head = rp.head, cnt = rp.count, pend = rp.pending;
  int bad = 0;
  if (head >= L) {
    head %= L;
    bad |= RSSM_ERR_POINTERS;
  }
  // commit-and-verify: the previous window's accepted drafts are committed first
  if (!APPEND && p.accepted != nullptr && pend > 0) commit_window(L, acc_prev, cnt, pend, bad);
  const int cmax = APPEND ? L - 1 : L - T;
  if (cnt > cmax) {
    cnt = cmax;
    bad |= RSSM_ERR_POINTERS;
  }
  if (pend != 0) bad |= RSSM_ERR_PENDING;
  const int c = cnt;
  const int E = c + T;
  const bool do_flush = APPEND ? (E == L) : (c + 2 * T > L);
  const int F = do_flush ? (APPEND ? E : c) : 0;
  const bool write_new = !(APPEND && do_flush);
  // logical entry held by physical slot sl (0 <= sl < L)
  auto logical = [&](int sl) { const int j = sl - head; return j < 0 ? j + L : j; };

  // ---- 4. the committed entries' ring keys (slot ps*16 + wave*4 + lane/16, 8
  //      columns per lane) and values (16 bytes per lane, by logical entry), now
  //      that the pointers are known: only the c entries in use are fetched, and
  //      they queue behind the checkpoint, which is needed first
  KC kr[PASSES][KQC];
#pragma unroll
  for (int ps = 0; ps < PASSES; ++ps) {
    const int sl = ps * 16 + wave * 4 + (lane >> 4);
#pragma unroll
    for (int ch = 0; ch < KQC; ++ch) kr[ps][ch] = zero_chunk<KC>();
    if (sl < L && logical(min(sl, L - 1)) < c) {
#pragma unroll
      for (int ch = 0; ch < KQC; ++ch)
        kr[ps][ch] = *reinterpret_cast<const KC*>(p.ring_k + (((size_t)rb * G + g) * L + sl) * N + sub * KPL +
                                                  ch * KQW);
    }
  }
  uint4 rv[RVP];
#pragma unroll
  for (int i = 0; i < RVP; ++i) {
    const int t = tid + i * kBlock;
    rv[i] = make_uint4(0, 0, 0, 0);
    if (t < c * (D / 8)) rv[i] = ld_u4(p.ring_v + ring_entry(rb, h, H, L, ring_slot(head, t / (D / 8), L), D) + (t % (D / 8)) * 8);
  }

  if constexpr (CONV) {
    // ---- 4b. the token's v, k, q from the conv (its operands arrive ahead of
    //      the checkpoint, and the ring loads are already on their way): window
    //      [s0, s1, s2, x], SiLU, bf16; shifted states out
    const int C = H * D + 2 * G * N;
    if (tid < NCQ) {
      const int lc = CPT * tid;
      // x states by their head; the group's B and C states spread over its heads
      // (1/hpg of them each, by the thread's first channel: the group's first
      // head writing them all ran 0.5 % slower); non-temporal, nothing in this
      // launch reads them again
      const bool owner = lc < D || ((lc - D) * hpg) / (2 * N) == h % hpg;
#pragma unroll
      for (int i = 0; i < CPR; ++i) {
        // the 6 state values of a pair (channel m owns 3m .. 3m + 2, oldest first), 2 tokens, 8 taps
        const v3u sp = cst[i];
        const uint32_t sv[6] = {sp.x & 0xffffu, sp.x >> 16, sp.y & 0xffffu, sp.y >> 16, sp.z & 0xffffu, sp.z >> 16};
        const uint32_t xv[2] = {cxv[i] & 0xffffu, cxv[i] >> 16};
        const uint4 wq = cwv[i];
        const uint32_t wv[8] = {wq.x & 0xffffu, wq.x >> 16, wq.y & 0xffffu, wq.y >> 16,
                                wq.z & 0xffffu, wq.z >> 16, wq.w & 0xffffu, wq.w >> 16};
        uint32_t o[2], ns[6];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const uint32_t win[4] = {sv[3 * m], sv[3 * m + 1], sv[3 * m + 2], xv[m]};
          o[m] = conv_silu_bf16(&wv[4 * m], win);
          ns[3 * m] = win[1];
          ns[3 * m + 1] = win[2];
          ns[3 * m + 2] = win[3];
        }
        *reinterpret_cast<uint32_t*>(&s_conv[lc + 2 * i]) = o[0] | (o[1] << 16);
        if (owner)
          __builtin_nontemporal_store(v3u{ns[0] | (ns[1] << 16), ns[2] | (ns[3] << 16), ns[4] | (ns[5] << 16)},
                                      reinterpret_cast<v3u*>(p.conv_out + ((size_t)rb * C + cch + 2 * i) * 3));
      }
    }
    __syncthreads();
#pragma unroll
    for (int ch = 0; ch < KQC; ++ch) {
      qm[0][ch] = *reinterpret_cast<const KC*>(&s_conv[D + N + sub * KPL + ch * KQW]);
      kin[0][ch] = *reinterpret_cast<const KC*>(&s_conv[D + sub * KPL + ch * KQW]);
    }
#pragma unroll
    for (int i = 0; i < NCP; ++i) {
      const int t = min(tid + i * kBlock, NCH - 1);
      newc[i] = *reinterpret_cast<const uint4*>(&s_conv[t < NEWV ? t * 8 : D + (t - NEWV) * 8]);
    }
  }

  // ---- 5. the new entries' values into their LDS slots (they are cached in the
  //      ring at the end)
#pragma unroll
  for (int i = 0; i < NCP; ++i) {
    const int t = tid + i * kBlock;
    if (t < NEWV) {
      const int sd = t / (D / 8), o = (t % (D / 8)) * 8;
      *reinterpret_cast<uint4*>(&s_v[ring_slot(head, c + sd, L) * D + o]) = newc[i];
    }
  }

  // ---- 6. wave 0: decay weights, stored by physical slot.  Lane l takes logical
  //      entry j = 63 - l, so products over the entries after j are prefix
  //      products over the lanes before l.
  if (wave == 0) {
    const int j = kWave - 1 - lane;                    // logical entry
    const int sj = ring_slot(head, min(j, L - 1), L);  // its physical slot
    const float dl_ring = __shfl(rec_l, kMetaSlot + sj, kWave);
    const float al_ring = expf(A_h * dl_ring);
    const float dtd = __shfl(dt_draft, min(max(j - c, 0), T - 1), kWave);
    const float dl_new = softplus_f32(dtd + dt_bias);
    const float al_new = expf(A_h * dl_new);
    const bool valid = j < E, cached = j < c;
    const float dl = valid ? (cached ? dl_ring : dl_new) : 0.f;
    const float al = valid ? (cached ? al_ring : al_new) : 1.f;
    const int wi = (j < L) ? sj : j;  // physical index this lane writes
#pragma unroll
    for (int sd = 0; sd < T; ++sd) {
      const int m = c + sd;  // last entry seen by draft sd
      float all;
      const float ex = prefix_product_excl(j <= m ? al : 1.f, &all);
      if (j < LCAP) s_w[sd][wi] = (j <= m) ? dl * ex : 0.f;
      if (lane == 0) s_abar[sd] = all;
    }
    {
      float all;
      const float ex = prefix_product_excl(j < F ? al : 1.f, &all);
      if (j < LCAP) s_fw[wi] = (j < F) ? dl * ex : 0.f;
      if (lane == 0) s_fabar = all;
    }
    if (j >= c && j < E) s_dtn[j - c] = dl;  // the new entries' step sizes
    if constexpr (!kQkLds && !CONV) {  // the query, for the output combine
      if (lane < 16) {
#pragma unroll
        for (int ch = 0; ch < KQC; ++ch) *reinterpret_cast<KC*>(&s_qk[sub * KPL + ch * KQW]) = qm[0][ch];
      }
    }
  }

  // ---- 7. all waves: k . q_s for every physical slot (16 lanes per slot); keys
  //      to fold staged by slot (zero rows for slots not folded).  The drafts'
  //      q and k come from registers at T = 1 and from LDS otherwise.
  const uint16_t* s_qv = CONV ? &s_conv[D + N] : s_qk;
  const uint16_t* s_kv = &s_qk[T * N];
  if constexpr (kQkLds) __syncthreads();
#pragma unroll
  for (int ps = 0; ps < PASSES; ++ps) {
    const int sl = ps * 16 + wave * 4 + (lane >> 4);
    const bool in_ring = sl < L;
    const int j = logical(min(sl, L - 1));
    KC kv[KQC];
#pragma unroll
    for (int ch = 0; ch < KQC; ++ch) kv[ch] = (in_ring && j < c) ? kr[ps][ch] : zero_chunk<KC>();
#pragma unroll
    for (int sd = 0; sd < T; ++sd)
      if (in_ring && j == c + sd)
#pragma unroll
        for (int ch = 0; ch < KQC; ++ch)
          kv[ch] = kQkLds ? *reinterpret_cast<const KC*>(&s_kv[sd * N + sub * KPL + ch * KQW]) : kin[0][ch];
    if (in_ring)
#pragma unroll
      for (int ch = 0; ch < KQC; ++ch)
        *reinterpret_cast<KC*>(&s_k[sl * N + sub * KPL + ch * KQW]) = (j < F) ? kv[ch] : zero_chunk<KC>();
#pragma unroll
    for (int sd = 0; sd < T; ++sd) {
      const KC* qs = kQkLds ? reinterpret_cast<const KC*>(&s_qv[sd * N + sub * KPL]) : qm[0];
      float dd = KL::dot(kv[0], qs[0]);
#pragma unroll
      for (int ch = 1; ch < KQC; ++ch) dd += KL::dot(kv[ch], qs[ch]);
      const float dv = reduce_quarter(dd);
      if (sub == 0) s_M[sd][sl] = dv;
    }
  }
  // the committed values into their LDS slots (waits for them only here)
#pragma unroll
  for (int i = 0; i < RVP; ++i) {
    const int t = tid + i * kBlock;
    if (t < c * (D / 8))
      *reinterpret_cast<uint4*>(&s_v[ring_slot(head, t / (D / 8), L) * D + (t % (D / 8)) * 8]) = rv[i];
  }
  __syncthreads();

  // ---- 9-10. the new entries cached in the ring unless this call empties it (v
  //      of this head, k by the group's first head), then this head's record
  //      rewritten as whole lines by wave 0: the new pointer word, A, and the step
  //      sizes with the new entries' in their slots.  Issued as the last stores
  //      of the kernel, after the outputs: with the state moved as whole lines,
  //      a one-token call storing them there instead of right after the barrier
  //      that ends phase 7 ran 2.7 % faster on non-flush launches (1.3 % over
  //      whole ring cycles, fused front-end 0.9 %), and 4 % faster than issuing
  //      them before that barrier; a verify stores them last as well (early, a
  //      round in which every request folds ran 2 % slower).
  auto store_entries_and_record = [&]() {
    if (write_new) {
      const bool k_owner = (h % hpg) == 0;
#pragma unroll
      for (int i = 0; i < NCP; ++i) {
        const int t = tid + i * kBlock;
        if (t < NEWV) {
          const int sd = t / (D / 8), o = (t % (D / 8)) * 8;
          *reinterpret_cast<uint4*>(p.ring_v + ring_entry(rb, h, H, L, ring_slot(head, c + sd, L), D) + o) = newc[i];
        } else if (k_owner && t < NCH) {
          const int tk = t - NEWV;
          const int sd = tk / (N / 8), o = (tk % (N / 8)) * 8;
          *reinterpret_cast<uint4*>(p.ring_k + (((size_t)rb * G + g) * L + ring_slot(head, c + sd, L)) * N + o) = newc[i];
        }
      }
    }
    if (wave == 0) {
      if (lane == 0 && h == 0) {
        flag_error(p.err, bad);
        if (p.flushed != nullptr) p.flushed[b] = do_flush ? 1 : 0;
      }
      const int keep = APPEND ? E : c;  // entries that stay committed unless flushed
      const unsigned long long nw =
          pack_ptr(do_flush ? ring_slot(head, F % L, L) : head, do_flush ? keep - F : keep, APPEND ? 0 : T);
      const int sl = lane - kMetaSlot;
      const int sd = (sl >= 0 && sl < L) ? logical(sl) - c : -1;
      float x = rec_l;
      if (lane == kMetaPtr) x = __uint_as_float(uint32_t(nw));
      if (lane == kMetaPtr + 1) x = __uint_as_float(uint32_t(nw >> 32));
      if (lane == kMetaA) x = A_h;
      if (write_new && sd >= 0 && sd < T) x = s_dtn[min(max(sd, 0), T - 1)];
      if (lane < MS) rec[lane] = x;
    }
  };

  // ---- 8. output-only route, fold when flushing (the checkpoint is needed here)
  float vj[RT][VJ];  // value of slot cq + 4m at this lane's rows, zero if not read
#pragma unroll
  for (int m = 0; m < VJ; ++m) {
    const int sl = cq + 4 * m;
    const bool used = sl < L && logical(min(sl, L - 1)) < E;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int row = (wave * RT + rt) * 16 + r;
      const float x = bf16_to_f32(s_v[min(sl, LCAP - 1) * D + row]);  // read unconditionally
      vj[rt][m] = used ? x : 0.f;
    }
  }
  if constexpr (T >= kMfmaCombineMinT) {
    // All drafts at once on the matrix cores, output tile = [16 state rows] x
    // [16 drafts] (drafts >= T are zero columns).  S_0 Q on v_mfma_f32_16x16x32_bf16
    // (lane l: A[l%16][8(l/16)..+7], B[8(l/16)..+7][l%16]): the state tile in
    // registers is the A operand as it stands, split into bf16 hi + lo (two MFMAs
    // per pair of column tiles), K index 8cq + e <-> column 32jj + 4cq + e and
    // 8cq + 4 + e <-> column 32jj + 16 + 4cq + e; B is the query of draft r at the
    // same columns, bf16 as stored.  Then the ring part V (W o M) accumulates on
    // top in fp32 (16x16x4): A = the values vj, B = w_{j,r} M_{j,r} for slot
    // j = cq + 4m.  Lane (cq, r) ends with y_r at rows 4cq .. 4cq + 3 of the tile.
    const bool draft = r < T;
    const int rd = min(r, T - 1);
    uint2 qb[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
      qb[ct] = draft ? *reinterpret_cast<const uint2*>(&s_qv[rd * N + ct * 16 + cq * 4]) : make_uint2(0, 0);
    float wm[VJ];
#pragma unroll
    for (int m = 0; m < VJ; ++m) wm[m] = draft ? s_w[rd][cq + 4 * m] * s_M[rd][cq + 4 * m] : 0.f;
    const float ab = draft ? s_abar[rd] : 0.f;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      v4f z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int jj = 0; jj < NCT / 2; ++jj) {
        settle_pair(st[rt][2 * jj], st[rt][2 * jj + 1]);
        const float4 s0 = st[rt][2 * jj], s1 = st[rt][2 * jj + 1];
        const float xs[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
        u32x4_t hi, lo;
        split_bf16x8(xs, hi, lo);
        const u32x4_t qv = {qb[2 * jj].x, qb[2 * jj].y, qb[2 * jj + 1].x, qb[2 * jj + 1].y};
        const bf16x8_t qbf = __builtin_bit_cast(bf16x8_t, qv);
        z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, hi), qbf, z, 0, 0, 0);
        z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, lo), qbf, z, 0, 0, 0);
      }
      z *= ab;
#pragma unroll
      for (int m = 0; m < VJ; ++m) {
        if (4 * m >= L) break;  // physical slots; uniform across the work-group
        z = mfma4(vj[rt][m], wm[m], z);
      }
      if (draft)
        *reinterpret_cast<float4*>(&s_y[rd * D + (wave * RT + rt) * 16 + cq * 4]) =
            make_float4(z[0], z[1], z[2], z[3]);
    }
  } else {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int row = (wave * RT + rt) * 16 + r;
      float dots[T];
#pragma unroll
      for (int sd = 0; sd < T; ++sd) dots[sd] = 0.f;
#pragma unroll
      for (int jj = 0; jj < NCT / 2; ++jj) {
        settle_pair(st[rt][2 * jj], st[rt][2 * jj + 1]);
#pragma unroll
        for (int ct = 2 * jj; ct < 2 * jj + 2; ++ct)
#pragma unroll
          for (int sd = 0; sd < T; ++sd)
            dots[sd] += dot4_bf16(st[rt][ct], *reinterpret_cast<const uint2*>(&s_qv[sd * N + ct * 16 + cq * 4]));
      }
#pragma unroll
      for (int sd = 0; sd < T; ++sd) {
        float part = s_abar[sd] * dots[sd];
#pragma unroll
        for (int m = 0; m < VJ; ++m) {
          const int sl = cq + 4 * m;
          part += s_w[sd][sl] * s_M[sd][sl] * vj[rt][m];  // zero for slots not read
        }
        part = reduce_row4(part);
        if ((sd & 3) == cq) s_y[sd * D + row] = part;
      }
    }
  }
  if (F > 0)
    fold_and_store<D, N, RT, NCT, VJ>(p.state0 + bh * D * N, st, s_fabar, s_k, s_fw, vj, L, wave, r, cq);

  // ---- 8b. the outputs, each draft's D values as whole lines (the waves hold 16
  //      rows each: staged through LDS, a quarter-line store per wave cost more)
  __syncthreads();
  for (int i = tid; i < T * D / 4; i += kBlock) {
    const int sd = i / (D / 4), o = (i % (D / 4)) * 4;
    const float4 f = *reinterpret_cast<const float4*>(&s_y[sd * D + o]);
    const size_t at = (((size_t)b * T + sd) * H + h) * D + o;
    if (p.y_bf16)
      *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.y) + at) =
          make_uint2(bf16_rne(f.x) | (bf16_rne(f.y) << 16), bf16_rne(f.z) | (bf16_rne(f.w) << 16));
    else
      st_f4(p.y + at, f);
  }

  store_entries_and_record();
}

}  // namespace rssm

namespace rssm_host {

using rssm::ReplayParams;

template <int D, int T, bool APPEND, bool CONV = false, int N = 128>
int launch_window(const ReplayParams& p, int B, void* stream) {
  const dim3 grid(B * p.H), block(rssm::kBlock);
  if (p.L <= 16) return launch(rssm::replay_window_kernel<D, N, T, APPEND, 16, CONV>, grid, block, stream, p);
  return launch(rssm::replay_window_kernel<D, N, T, APPEND, 32, CONV>, grid, block, stream, p);
}

// Verify launchers for T = 1..4 and T = 5..8 (n = 128) live in their own
// translation units, and so do the append, verify and fused front-end launchers
// of n = 64 and n = 256 (T = 0 selects the append).
__attribute__((visibility("hidden"))) int launch_replay_verify_lo(int T, int D, const ReplayParams& p, int B, void* stream);
__attribute__((visibility("hidden"))) int launch_replay_verify_hi(int T, int D, const ReplayParams& p, int B, void* stream);
__attribute__((visibility("hidden"))) int launch_replay_n64(int T, int D, const ReplayParams& p, int B, void* stream);
__attribute__((visibility("hidden"))) int launch_replay_n256(int T, int D, const ReplayParams& p, int B, void* stream);
__attribute__((visibility("hidden"))) int launch_replay_conv_n64(int D, const ReplayParams& p, int B, void* stream);
__attribute__((visibility("hidden"))) int launch_replay_conv_n256(int D, const ReplayParams& p, int B, void* stream);

}  // namespace rssm_host
