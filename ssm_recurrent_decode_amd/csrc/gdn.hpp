// Gated DeltaNet ReplaySSM verify kernel and its launcher, shared by the
// translation units that instantiate it.
//
// Method: "ReplaySSM: Cache SSM Inputs, Not State" -- appendix, GDN standard
// decode (the correction u is cached so the update becomes S_t = alpha_t S_{t-1}
// + u_t k_t^T) and GDN speculative decoding (all T corrections of a window from
// one strictly lower-triangular T x T solve).
#pragma once

#include "common.hpp"

namespace rssm {

struct GdnReplayParams {
  float* state0;
  float* ring_u;       // [B, H, L, D] fp32
  uint16_t* ring_k;    // [B, G, L, N]
  float* meta;         // [B, H, meta_words(L)] per-head ring records (alpha per slot)
  int32_t* err;
  const uint16_t* v;   // [B, T, H, D]
  const uint16_t* k;   // [B, T, G, N]
  const uint16_t* q;   // [B, T, G, N]
  const float* g;      // [B, T, H]
  const float* beta;   // [B, T, H]
  float* y;            // [B, T, H, D]
  int32_t* flushed;
  const int32_t* mask;
  const int32_t* accepted;  // commit-and-verify: the previous window's accepted drafts, or null
  const int32_t* slots;  // pool row per batch entry, or null
  int rows;
  int y_bf16;          // outputs stored as bf16
  int u_bf16;          // ring corrections cached as bf16 [B, H, L, D]
  int H, G, L;
};

// One verify round of T drafts, one work-group of four waves per (request, head).
// Entries in logical order: the c committed ones (ring), then the T drafts.
// APPEND (T == 1, standard decode): the token is committed in the same call
// (count <- c + 1, pending stays 0) and the ring is flushed when the append
// fills it, the new entry included (S_0 <- prod alpha S_0 + sum_j w_j u_j k_j^T
// over all L entries, after the new correction is known).
//   committed-state readouts  S_c x = abar S_0 x + sum_{j<c} w_j u_j (k_j . x),
//     abar = prod_{i<c} alpha_i,  w_j = prod_{j<i<c} alpha_i,  x in {k_s, q_s};
//   R_s = beta_s (v_s - gamma_s S_c k_s),  gamma_s = prod_{s'<=s} alpha'_s';
//   u_s = R_s - sum_{s'<s} beta_s (prod_{s'<i<=s} alpha'_i) (k_s . k_s') u_s'
//     (forward substitution of the strictly lower-triangular system);
//   y_s = gamma_s S_c q_s + sum_{s'<=s} (prod_{s'<i<=s} alpha'_i) (k_s' . q_s) u_s';
//   the drafts' (u, k, alpha') are cached in their ring slots; when c + 2T > L
//   the committed entries are folded first: S_0 <- abar S_0 + sum_j w_j u_j k_j^T.
//
// As in the Mamba-2 window kernel, the ring record (pointer word and the decays
// of all L slots) and every small operand -- the 2T readout vectors and the draft
// values (16 bytes per lane into LDS), the gates and betas -- are requested
// before the checkpoint tiles, and the ring keys and corrections of the c
// committed entries only (16 bytes per lane into LDS) right after them, once the
// pointer word is in; the weights proceed while the checkpoint is in flight.  The 2T readouts S_0 x run on
// the matrix cores from the state registers; the fold (when flushing) follows
// from the same registers; the per-row solve runs one thread per row after that.
// Waves per SIMD the register budget is sized for.  At n = 128: four (128
// registers) with a ring of up to 16 slots; a 32-slot ring keeps twice the
// committed corrections and fold operands live, so three (168) where that fits
// without spilling to scratch, two (256) or one (512, accumulation registers
// included) for the widest windows.  n = 64 halves the checkpoint registers, n =
// 256 doubles them (d = 128, n = 256: 128 registers for the checkpoint alone).
// The build rejects any kernel that spills.
template <int D, int N, int T, int LCAP>
constexpr int gdn_waves_per_simd() {
  if (N == 64) return LCAP == 16 ? (T <= 7 ? 5 : 4) : (D == 64 || T <= 2 ? 4 : 3);
  if (N == 256) return D == 64 ? (LCAP == 16 ? 4 : 3) : 2;
  if (LCAP == 16) return 4;
  if (D == 64) return T <= 5 ? 3 : 2;
  return T <= 1 ? 3 : (T <= 6 ? 2 : 1);
}

template <int D, int N, int T, int LCAP, bool APPEND = false>
__global__ __launch_bounds__(kBlock, (gdn_waves_per_simd<D, N, T, LCAP>())) void gdn_verify_kernel(GdnReplayParams p) {
  static_assert(N == 64 || N == 128 || N == 256, "keys and queries: 16 lanes of n / 16 values");
  static_assert(!APPEND || T == 1, "append-decode is one token");
  static_assert(2 * T <= 16, "readout vectors must fit one MFMA M axis");
  static_assert(D <= kBlock, "one thread per state row in the solve");
  static_assert(LCAP == 16 || LCAP == 32, "ring capacity bound");
  constexpr int NCT = N / 16;
  constexpr int RT = D / (16 * kWavesPerBlock);
  constexpr int NV = 2 * T;               // readout vectors: k_0..k_{T-1}, q_0..q_{T-1}
  constexpr int VJ = LCAP / 4;            // physical slots per lane in the fold
  constexpr int PASSES = LCAP / 16;       // inner-product passes of 16 slots
  constexpr int XC = NV * N / 8;          // 16-byte chunks of the readout vectors
  constexpr int VC = T * D / 8;           // ... of the draft values
  constexpr int XVP = (XC + VC + kBlock - 1) / kBlock;
  constexpr int UC = LCAP * D / 4;        // ... of the ring corrections (fp32)
  constexpr int UP = (UC + kBlock - 1) / kBlock;
  using KL = KeyLanes<N>;  // a key or readout vector over 16 lanes, KQC chunks of KQW values each
  using KC = typename KL::Chunk;
  constexpr int KQC = KL::C, KQW = KL::W, KPL = N / 16;
  __shared__ float s_Z[NV][D];            // (S_0 x_v)[row]
  __shared__ float s_M[NV][LCAP];         // k_slot . x_v by physical slot
  __shared__ float s_w[LCAP];             // w_j by physical slot, zero if not committed
  __shared__ float s_abar;
  __shared__ float s_fw[APPEND ? LCAP : 1];  // append flush: weights over all E entries
  __shared__ float s_fabar;
  __shared__ float s_alpha_d[T];          // draft decays alpha'_s
  __shared__ float s_beta[T];
  __shared__ __attribute__((aligned(16))) uint16_t s_x[NV * N];     // readout vectors
  __shared__ __attribute__((aligned(16))) uint16_t s_vd[T * D];     // draft values
  __shared__ __attribute__((aligned(16))) uint16_t s_k[LCAP * N];   // keys to fold by slot
  __shared__ __attribute__((aligned(16))) float s_u[LCAP * D];      // corrections by slot

  const int H = p.H, G = p.G, L = p.L;
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int b = wg / H, h = wg - b * H, hpg = H / G, g = h / hpg;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, cq = lane >> 4, sub = lane & 15;
  const int rb = pool_row(p.slots, p.rows, b, p.err, tid == 0 && h == 0);  // request's row
  if (rb < 0) return;                 // padding or outside the pool: whole work-group
  const size_t bh = (size_t)rb * H + h;  // per-(row, head) checkpoint, ring and record

  // ---- 1. this head's copy of the pointer word and every small operand
  const int MS = meta_words(L);
  float* rec = p.meta + bh * MS;  // this head's ring record
  // (both read per lane, so that the checkpoint loads are issued before they arrive)
  const int z0 = opaque_zero();
  const unsigned long long word = *reinterpret_cast<const unsigned long long*>(rec + kMetaPtr + z0);
  const int acc_prev = (!APPEND && p.accepted != nullptr) ? p.accepted[b + z0] : 0;
  uint4 xvc[XVP];  // readout vectors (k drafts, then q drafts), then the draft values
#pragma unroll
  for (int i = 0; i < XVP; ++i) {
    const int t = min(tid + i * kBlock, XC + VC - 1);
    const uint16_t* src;
    if (t < XC) {
      const int v = t / (N / 8), o = (t % (N / 8)) * 8;
      src = (v < T) ? p.k + (((size_t)b * T + v) * G + g) * N + o
                    : p.q + (((size_t)b * T + (v - T)) * G + g) * N + o;
    } else {
      const int tv = t - XC;
      src = p.v + (((size_t)b * T + tv / (D / 8)) * H + h) * D + (tv % (D / 8)) * 8;
    }
    xvc[i] = ld_u4(src);
  }
  // the whole record (decays of every slot), the drafts' gates and betas: read by
  // every wave, though only wave 0 uses them (behind a wave-0 branch the compiler
  // computed the gates' exponentials there, and wave 0 waited for them before
  // issuing its checkpoint loads)
  const float rec_l = rec[min(lane, MS - 1)];
  const float gd = p.g[((size_t)b * T + min(lane, T - 1)) * H + h];
  const float bt = p.beta[((size_t)b * T + min(lane, T - 1)) * H + h];

  // ---- 2. the checkpoint, last (the scheduler may not hoist it above the rest)
  __builtin_amdgcn_sched_barrier(0);
  float* S0 = p.state0 + bh * D * N;
  float4 st[RT][NCT];  // line arrangement; each pair settled where the readouts first use it
  load_state_lines<N, RT, NCT>(st, S0, wave, r, cq);

  // ---- 3. small operands into LDS; pointers, clamped into range
#pragma unroll
  for (int i = 0; i < XVP; ++i) {
    const int t = tid + i * kBlock;
    if (t < XC) *reinterpret_cast<uint4*>(&s_x[t * 8]) = xvc[i];
    else if (t < XC + VC) *reinterpret_cast<uint4*>(&s_vd[(t - XC) * 8]) = xvc[i];
  }
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
  // verify: early flush of the c committed entries; append: flush when full
  const bool do_flush = APPEND ? (E == L) : (c + 2 * T > L);
  const int F = do_flush ? (APPEND ? E : c) : 0;  // entries folded
  const bool write_new = !(APPEND && do_flush);
  // logical entry held by physical slot sl (0 <= sl < L)
  auto logical = [&](int sl) { const int j = sl - head; return j < 0 ? j + L : j; };

  // the committed entries' ring keys (slot ps*16 + wave*4 + lane/16, 8 columns per
  // lane) and corrections (16 bytes per lane, by logical entry), now that the
  // pointers are known: only the c entries in use, queued behind the checkpoint
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
  const int cpe = p.u_bf16 ? D / 8 : D / 4;  // 16-byte chunks per cached correction
  uint4 uc[UP];
#pragma unroll
  for (int i = 0; i < UP; ++i) {
    const int t = tid + i * kBlock;
    uc[i] = make_uint4(0, 0, 0, 0);
    if (t < c * cpe) {
      const size_t e = ring_entry(rb, h, H, L, ring_slot(head, t / cpe, L), D);
      uc[i] = p.u_bf16 ? ld_u4(reinterpret_cast<const uint16_t*>(p.ring_u) + e + (t % cpe) * 8)
                       : *reinterpret_cast<const uint4*>(p.ring_u + e + (t % cpe) * 4);
    }
  }

  // ---- 4. wave 0: decay weights of the committed entries (lane l takes logical
  //      entry 63 - l, so products over later entries are prefix products), the
  //      draft decays and betas, the drafts' decays cached in the ring
  if (wave == 0) {
    const int j = kWave - 1 - lane;
    const int sj = ring_slot(head, min(j, L - 1), L);
    const float al = __shfl(rec_l, kMetaSlot + sj, kWave);
    float all;
    const float ex = prefix_product_excl(j < c ? al : 1.f, &all);
    if (j < LCAP) s_w[(j < L) ? sj : j] = (j < c) ? ex : 0.f;
    if (lane == 0) s_abar = all;
    if constexpr (APPEND) {  // fold weights over the c committed entries and the new one
      const float af = (j < c) ? al : expf(gd);
      float allf;
      const float exf = prefix_product_excl(j < F ? af : 1.f, &allf);
      if (j < LCAP) s_fw[(j < L) ? sj : j] = (j < F) ? exf : 0.f;
      if (lane == 0) s_fabar = allf;
    }
    if (lane < T) {
      s_alpha_d[lane] = expf(gd);
      s_beta[lane] = bt;
    }
  }
  __syncthreads();

  // ---- 5. all waves: k_slot . x_v for every physical slot (16 lanes per slot);
  //      keys to fold staged by slot; the drafts' keys cached by the group owner
#pragma unroll
  for (int ps = 0; ps < PASSES; ++ps) {
    const int sl = ps * 16 + wave * 4 + (lane >> 4);
    const bool in_ring = sl < L;
    const int j = logical(min(sl, L - 1));
    const int sd = j - c;
    KC kv[KQC];
#pragma unroll
    for (int ch = 0; ch < KQC; ++ch) {
      kv[ch] = (in_ring && j < c) ? kr[ps][ch] : zero_chunk<KC>();
      if (in_ring && sd >= 0 && sd < T) kv[ch] = *reinterpret_cast<const KC*>(&s_x[sd * N + sub * KPL + ch * KQW]);
      if (in_ring)
        *reinterpret_cast<KC*>(&s_k[sl * N + sub * KPL + ch * KQW]) = (j < F) ? kv[ch] : zero_chunk<KC>();
    }
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      float dd = 0.f;
#pragma unroll
      for (int ch = 0; ch < KQC; ++ch)
        dd += KL::dot(kv[ch], *reinterpret_cast<const KC*>(&s_x[v * N + sub * KPL + ch * KQW]));
      const float d = reduce_quarter(dd);
      if (sub == 0) s_M[v][sl] = d;
    }
  }
  if (write_new && h % hpg == 0) {
    for (int t = tid; t < T * (N / 8); t += kBlock) {
      const int sd = t / (N / 8), o = (t % (N / 8)) * 8;
      *reinterpret_cast<uint4*>(p.ring_k + (((size_t)rb * G + g) * L + ring_slot(head, c + sd, L)) * N + o) =
          *reinterpret_cast<const uint4*>(&s_x[sd * N + o]);
    }
  }
  // the committed corrections into their LDS slots (waits for them only here)
#pragma unroll
  for (int i = 0; i < UP; ++i) {
    const int t = tid + i * kBlock;
    if (t < c * cpe) {
      float* dst = &s_u[ring_slot(head, t / cpe, L) * D];
      if (p.u_bf16) {
        const int o = (t % cpe) * 8;
        *reinterpret_cast<float4*>(dst + o) =
            make_float4(bf16_lo(uc[i].x), bf16_hi(uc[i].x), bf16_lo(uc[i].y), bf16_hi(uc[i].y));
        *reinterpret_cast<float4*>(dst + o + 4) =
            make_float4(bf16_lo(uc[i].z), bf16_hi(uc[i].z), bf16_lo(uc[i].w), bf16_hi(uc[i].w));
      } else {
        *reinterpret_cast<uint4*>(dst + (t % cpe) * 4) = uc[i];
      }
    }
  }
  __syncthreads();

  // ---- 6. readouts Z = S_0 [K|Q] on the matrix cores (v_mfma_f32_16x16x32_bf16):
  //      A[m][k] = x_m[col] (bf16 as stored), B[k][nn] = S_0[row nn][col] split into
  //      bf16 hi + lo (two MFMAs per pair of column tiles; K index 8cq + e <->
  //      column 32jj + 4cq + e, 8cq + 4 + e <-> 32jj + 16 + 4cq + e); lane (r, cq)
  //      ends with Z[4cq+i][row r of the tile].  The committed entries' part of
  //      the committed-state readouts accumulates on top in fp32
  //      (v_mfma_f32_16x16x4_f32, K = ring slots): Z <- abar Z + (W o M) U, with
  //      A[v][slot] = w_slot (k_slot . x_v) and B[slot][row] = u_slot[row], so the
  //      per-row phase below starts from S_c x_v directly.
  uint2 xq[NCT];  // this lane's readout vector x_r at the columns of each tile
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
    xq[ct] = (r < NV) ? *reinterpret_cast<const uint2*>(&s_x[r * N + ct * 16 + cq * 4]) : make_uint2(0, 0);
  const float abar = s_abar;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int jj = 0; jj < NCT / 2; ++jj) {
      settle_pair(st[rt][2 * jj], st[rt][2 * jj + 1]);
      const float4 s0 = st[rt][2 * jj], s1 = st[rt][2 * jj + 1];
      const float xs[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
      u32x4_t hi, lo;
      split_bf16x8(xs, hi, lo);
      const u32x4_t xv = {xq[2 * jj].x, xq[2 * jj].y, xq[2 * jj + 1].x, xq[2 * jj + 1].y};
      const bf16x8_t xbf = __builtin_bit_cast(bf16x8_t, xv);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xbf, __builtin_bit_cast(bf16x8_t, hi), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xbf, __builtin_bit_cast(bf16x8_t, lo), acc, 0, 0, 0);
    }
    acc *= abar;
    const int row = (wave * RT + rt) * 16 + r;
#pragma unroll
    for (int m = 0; m < VJ; ++m) {
      if (4 * m >= L) break;  // physical slots; uniform across the work-group
      const int sl = 4 * m + cq;  // A: w_sl (k_sl . x_r), B: u_sl at this lane's row
      const bool cm = sl < L && logical(min(sl, L - 1)) < c;
      const float a = (cm && r < NV) ? s_w[sl] * s_M[min(r, NV - 1)][sl] : 0.f;
      acc = mfma4(a, cm ? s_u[sl * D + row] : 0.f, acc);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (4 * cq + i < NV) s_Z[4 * cq + i][row] = acc[i];
  }

  // ---- 7. early flush of the committed entries (from the same registers)
  if (!APPEND && do_flush) {
    float uf[RT][VJ];  // correction of slot cq + 4m at this lane's rows, zero if not folded
#pragma unroll
    for (int m = 0; m < VJ; ++m) {
      const int sl = cq + 4 * m;
      const bool used = sl < L && logical(min(sl, L - 1)) < c;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        uf[rt][m] = used ? s_u[min(sl, LCAP - 1) * D + (wave * RT + rt) * 16 + r] : 0.f;
    }
    fold_and_store<D, N, RT, NCT, VJ>(S0, st, s_abar, s_k, s_w, uf, L, wave, r, cq);
  }
  __syncthreads();

  // ---- 8. per row: the committed-state readouts S_c x_v (from step 6),
  //      corrections by forward substitution, outputs, the corrections cached
  //      in the ring
  const int rho = tid;
  if (rho < D) {
    float sh[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) sh[v] = s_Z[v][rho];
    int dslot[T];  // physical slots of the drafts
#pragma unroll
    for (int sd = 0; sd < T; ++sd) dslot[sd] = ring_slot(head, c + sd, L);
    float gamma[T];
    {
      float gm = 1.f;
#pragma unroll
      for (int sd = 0; sd < T; ++sd) {
        gm *= s_alpha_d[sd];
        gamma[sd] = gm;
      }
    }
    float u[T];
#pragma unroll
    for (int sd = 0; sd < T; ++sd) {
      const float bs = s_beta[sd];
      float acc = bs * (bf16_to_f32(s_vd[sd * D + rho]) - gamma[sd] * sh[sd]);  // R_s
      float ratio = 1.f;                                                       // prod_{s'<i<=s} alpha'_i
#pragma unroll
      for (int sp = sd - 1; sp >= 0; --sp) {
        ratio *= s_alpha_d[sp + 1];
        acc -= bs * ratio * s_M[sd][dslot[sp]] * u[sp];  // A_{s,s'} u_{s'}
      }
      u[sd] = acc;
    }
#pragma unroll
    for (int sd = 0; sd < T; ++sd) {
      float acc = gamma[sd] * sh[T + sd];
      float ratio = 1.f;
#pragma unroll
      for (int sp = sd; sp >= 0; --sp) {
        if (sp < sd) ratio *= s_alpha_d[sp + 1];
        acc += ratio * s_M[T + sd][dslot[sp]] * u[sp];
      }
      const size_t at = (((size_t)b * T + sd) * H + h) * D + rho;
      if (p.y_bf16) reinterpret_cast<uint16_t*>(p.y)[at] = (uint16_t)bf16_rne(acc);
      else p.y[at] = acc;
      // the correction as cached (rounded when the ring holds bf16); this call's
      // outputs above used it unrounded
      const uint32_t ub = bf16_rne(u[sd]);
      const size_t ua = ring_entry(rb, h, H, L, dslot[sd], D) + rho;
      if (write_new) {
        if (p.u_bf16) reinterpret_cast<uint16_t*>(p.ring_u)[ua] = (uint16_t)ub;
        else p.ring_u[ua] = u[sd];
      } else {
        s_u[dslot[sd] * D + rho] = p.u_bf16 ? bf16_to_f32(ub) : u[sd];  // append filling the ring: folded below
      }
    }
  }

  // ---- 8b. append that fills the ring: fold all E entries, the new one included
  if constexpr (APPEND) {
    if (do_flush) {
      __syncthreads();
      float uf[RT][VJ];
#pragma unroll
      for (int m = 0; m < VJ; ++m) {
        const int sl = cq + 4 * m;
        const bool used = sl < L;  // every slot holds one of the E = L entries
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const float x = s_u[min(sl, LCAP - 1) * D + (wave * RT + rt) * 16 + r];
          uf[rt][m] = used ? x : 0.f;
        }
      }
      fold_and_store<D, N, RT, NCT, VJ>(S0, st, s_fabar, s_k, s_fw, uf, L, wave, r, cq);
    }
  }

  // ---- 9. this head's record rewritten as whole lines by wave 0: the new pointer
  //      word and the decays with the drafts' in their slots
  if (wave == 0) {
    if (lane == 0 && h == 0) {
      flag_error(p.err, bad);
      if (p.flushed != nullptr) p.flushed[b] = do_flush ? 1 : 0;
    }
    const unsigned long long nw =
        APPEND ? pack_ptr(do_flush ? (head + E) % L : head, do_flush ? 0 : E, 0)
               : pack_ptr(do_flush ? (head + c) % L : head, do_flush ? 0 : c, T);
    const int sl = lane - kMetaSlot;
    const int sd = (sl >= 0 && sl < L) ? logical(sl) - c : -1;
    float x = rec_l;
    if (lane == kMetaPtr) x = __uint_as_float(uint32_t(nw));
    if (lane == kMetaPtr + 1) x = __uint_as_float(uint32_t(nw >> 32));
    if (write_new && sd >= 0 && sd < T) x = s_alpha_d[min(max(sd, 0), T - 1)];
    if (lane < MS) rec[lane] = x;
  }
}

}  // namespace rssm

namespace rssm_host {

using rssm::GdnReplayParams;

template <int D, int T, bool APPEND = false, int N = 128>
int launch_gdn_window(const GdnReplayParams& p, int B, void* stream) {
  const dim3 grid(B * p.H), block(rssm::kBlock);
  if (p.L <= 16) return launch(rssm::gdn_verify_kernel<D, N, T, 16, APPEND>, grid, block, stream, p);
  return launch(rssm::gdn_verify_kernel<D, N, T, 32, APPEND>, grid, block, stream, p);
}

// Verify launchers for T = 1..4 and T = 5..8 (n = 128) live in their own
// translation units, and so do the append and verify launchers of n = 64 and
// n = 256 (T = 0 selects the append).
__attribute__((visibility("hidden"))) int launch_gdn_verify_lo(int T, int D, const GdnReplayParams& p, int B, void* stream);
__attribute__((visibility("hidden"))) int launch_gdn_verify_hi(int T, int D, const GdnReplayParams& p, int B, void* stream);
__attribute__((visibility("hidden"))) int launch_gdn_n64(int T, int D, const GdnReplayParams& p, int B, void* stream);
__attribute__((visibility("hidden"))) int launch_gdn_n256(int T, int D, const GdnReplayParams& p, int B, void* stream);

}  // namespace rssm_host
