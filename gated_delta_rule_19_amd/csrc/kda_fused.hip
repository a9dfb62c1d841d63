// KDA chunked prefill with chunk prep and state carry fused in one kernel
// (bf16 inputs, fp32 state and accumulation): one workgroup per (sequence,
// head) carries all 128 state columns, and each chunk's operands are built
// in LDS by the same workgroup while it carries the state through the
// previous chunk.  Only the layer's own inputs and outputs touch HBM.
//
// The mathematics is the FlashKDA chunk form of "Kimi K3 的架構"
// (hao.cnyes.com) §六, with the 16-token reference points that the decay's
// lower bound allows ("Kimi K3.1 Pro 架构完全拆解" §3.2).  With G the
// inclusive cumulative log-decay from the chunk start, p_I = G before token
// tile I, G_loc = G - p_I, tot_I = the tile's total and G_C the chunk total:
//   Q_loc = q e^{G_loc},  K_loc = k e^{G_loc},  K_st = k e^{-G_loc}   (<= e^80 |k|)
//   K_rs  = K_st e^{tot_I} = k e^{p_{I+1} - G}                        (<= |k|)
//   Q_decay = Q_loc e^{p_I},  K_decay = K_loc e^{p_I},  K_restore = K_rs e^{G_C - p_{I+1}}
//   L_IJ = Diag(beta) K_loc,I B_IJ^T,  M_IJ = Q_loc,I B_IJ^T   (J <= I)
//   with B_II = K_st,I and, for J < I, B_IJ = K_rs,J e^{p_I - p_{J+1}} = k_t e^{p_I - G_t}
// (every factor and partial product is at most 1 in size except K_st's, so
// a result underflows only where the exact value is negligible).
//
// The state step per chunk is the pages' U = INV Diag(beta)(V - K_decay S),
// O = Q_decay S + M_qk U, S = Diag(a_last) S + K_restore^T U, with INV =
// (I + L)^-1 applied by block forward substitution over the four 16-token
// tiles (any exact method gives the same unique result):
//   U_I = D_I^-1 (Diag(beta_I)(V_I - W_I) - sum_{J<I} L_IJ U_J),  D_I = I + L_II,
// where D_I^-1 comes from the Neumann product (I - N)(I + N^2)(I + N^4)(I + N^8)
// of the strictly lower N = L_II (N^16 = 0).
//
// Workgroup of 8 waves, two per SIMD:
//   waves 0-3, state: wave w carries state columns 32 w .. 32 w + 31 (two
//     16-column MFMA tiles) through the chunks, S in MFMA accumulators.
//     After its chunk step it also inverts D_w of the chunk being prepared:
//     a chain of dependent MFMAs that would otherwise sit on the prep waves'
//     path, which is the longer one;
//   waves 4-7, prep: wave 4 + I owns token tile I of the chunk being
//     prepared.  Lane (lr, lg) = (lane % 16, lane / 16) holds token 16 I + lr
//     and, for k-step s, channels 32 s + 8 lg .. + 7: one 16-byte load per
//     input and k-step, and the MFMA A-fragment layout.
// Step k: the prep waves build chunk k's operands while the state waves
// consume chunk k - 1's; one workgroup barrier ends each step.  The prep
// waves also scan chunk k + 1's decay within step k, and once they have met
// (every tile total written) the state waves, whose path is the shorter,
// turn the totals into the per-channel factors, state wave w those of token
// tile w: chunk k + 1's elementwise work starts as soon as step k + 1 does.
// Q_decay, K_decay, M_qk and the L and
// D^-1 blocks, which the state waves read early in a step, have one LDS
// copy: the prep waves overwrite them only after every state wave has
// counted itself done with the previous chunk's (LDS counters, bounded
// waits).  K_restore (token-major; the state waves read it transposed with
// gfx950's transposing LDS reads), beta and a_last, read late, have two
// copies by chunk parity.  The prep waves meet once per step, before the off-
// diagonal tile pairs (every tile's K_rs and tile totals written).  A
// wave on the same SIMD as MFMA work loses VALU issue to it, so the work
// is spread to keep each SIMD's share even rather than to keep MFMA away
// from the VALU-bound prep.
//
// State row order: accumulator row p holds channel kperm(p) (kda_internal.h),
// so two stacked accumulator tiles packed together are the B operand of the
// channel-contracting products with channels in natural order.  Token
// columns of the token-contracting operands (M_qk, K_restore^T) are in kperm
// order to match U packed the same way.  o is computed transposed (the same
// fragments with the operand roles swapped), so that a lane holds four
// adjacent output columns of one token and stores them as one 8-byte piece.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int kFusedThreads = 512;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kLdN = 20; // fp32 row stride of the N blocks

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// acc(16x16) += A(16x16) B(16x16) on v_mfma_f32_16x16x16_bf16: lane (lr, lg)
// gives A[lr][4 lg .. + 3] and B[4 lg .. + 3][lr], the accumulator layout of B.
__device__ __forceinline__ f32x4 mma16(f32x4 acc, bf16x4 a, bf16x4 b) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                   __builtin_bit_cast(s16x4, b), acc, 0, 0, 0);
}

__device__ __forceinline__ bf16x4 pack4(const f32x4 &x) {
  bf16x4 v;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    v[i] = static_cast<bf16>(x[i]);
  return v;
}

// A B in the column layout for 16 x 16 fp32 blocks (a: A in the row layout,
// b: B in the column layout, as mm16_rr), with the four K = 4 steps in two
// independent accumulators so that the chain of dependent MFMAs is half as
// long; c is added.
__device__ __forceinline__ f32x4 mm16_split(const f32x4 c, const f32x4 a, const f32x4 b) {
  f32x4 x = c, y = {0.f, 0.f, 0.f, 0.f};
  x = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], x, 0, 0, 0);
  y = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], y, 0, 0, 0);
  x = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], x, 0, 0, 0);
  y = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], y, 0, 0, 0);
  return x + y;
}

// One chunk's operands in LDS.  The bf16 MFMA A operands of the state step
// are stored as fragment blocks: 1 KiB per (16-row tile, 32-wide k-step),
// lane l's 16 bytes at 16 l, so a fragment read is 64 consecutive 16-byte
// pieces.  The 16 x 16 operands of the substitution are 512-byte blocks,
// lane l's 8 bytes at 8 l.
struct RecOnce {     // one copy (read early in a step)
  bf16 qd[16][512];  // Q_decay, block 4 tt + s
  bf16 kd[16][512];  // K_decay, block 4 tt + s
  bf16 mqk[8][512];  // M_qk, block 2 tt + s'
  bf16 lo[6][256];   // L_IJ, J < I, at off_pair(I, J)
  bf16 dn[4][256];   // -(I + L_II)^-1
};
// K_restore's row stride in LDS, in elements: 32 elements of padding put the
// four token rows of one transposed read in different banks
constexpr int kKrLd = kD + 32;
struct RecTwice {      // two copies by chunk parity (read late in a step)
  bf16 kr[kC][kKrLd];  // K_restore, token-major (channels in order)
  float beta[kC];
  float al[kD];      // a_last by state row
};

struct PrepScratch {
  float tot[4][kD];        // tile totals of g (log2 units) per channel
  float fac[4][5][kD];     // per prep wave: its per-channel factors
  bf16 krs[3][4][512];     // K_rs of token tiles 0..2, fragment blocks per k-step
  bf16 bsc[3][4][512];     // B_20, B_30, B_31 (K_rs,J scaled to tile I's reference point)
  bf16 t3k[4][512];        // K_loc of token tile 3, fragment blocks per k-step
  bf16 t3q[4][512];        // Q_loc of token tile 3
  float nmat[4][16][kLdN]; // N of each token tile, fp32, row-major
  float alast[kD];         // a_last of the chunk being prepared, by channel
};

struct FusedSmem {
  RecOnce a;
  RecTwice b[2];
  PrepScratch ps;
  bf16 vst[4][kC * 32]; // each state wave's 64 x 32 slice of v (vst_off)
  float ored[4][kC];    // output norm: each state wave's sums of o^2 per token
  int meet;             // prep waves' arrivals at their meetings
  int q_done;           // state waves done reading Q_decay, K_decay
  int m_done;           // state waves done reading M_qk, L, D^-1
  int n_ready;          // prep waves' N blocks written
  int o_red;            // state waves' output-norm sums written
};
static_assert(sizeof(FusedSmem) <= 160 * 1024, "fused prefill LDS");

__device__ __forceinline__ int off_pair(int I, int J) { return I * (I - 1) / 2 + J; }

// Token tile I's factor rows from the four tile totals (two channels per
// lane): 0 e^{p_I}, 1 e^{tot_I}, 2 e^{G_C - p_{I+1}}, and the scales of the
// non-adjacent pair operands built from that tile (tile 0: 3 e^{tot_1} for
// B_20, 4 e^{tot_1 + tot_2} for B_30; tile 1: 3 e^{tot_2} for B_31); with
// tile 0 also a_last by channel.  I is wave-uniform.
__device__ __forceinline__ void tile_factors(PrepScratch &P, int I, int lane) {
  const int c0 = 2 * lane;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int c = c0 + e;
    const float t0 = P.tot[0][c], t1 = P.tot[1][c], t2 = P.tot[2][c], t3 = P.tot[3][c];
    const float pI = I == 0 ? 0.f : (I == 1 ? t0 : (I == 2 ? t0 + t1 : t0 + t1 + t2));
    const float tI = I == 0 ? t0 : (I == 1 ? t1 : (I == 2 ? t2 : t3));
    const float gC = t0 + t1 + t2 + t3;
    P.fac[I][0][c] = __builtin_amdgcn_exp2f(pI);           // e^{p_I} <= 1
    P.fac[I][1][c] = __builtin_amdgcn_exp2f(tI);           // e^{tot_I} in [e^-80, 1]
    P.fac[I][2][c] = __builtin_amdgcn_exp2f(gC - pI - tI); // e^{G_C - p_{I+1}} <= 1
    if (I == 0) {
      P.fac[0][3][c] = __builtin_amdgcn_exp2f(t1);
      P.fac[0][4][c] = __builtin_amdgcn_exp2f(t1 + t2);
      P.alast[c] = __builtin_amdgcn_exp2f(gC);
    }
    if (I == 1)
      P.fac[1][3][c] = __builtin_amdgcn_exp2f(t2);
  }
}

// LDS synchronisation, written out: the compiler's own fences and barriers
// would also wait for the LDS DMA of the next chunk's v that each state wave
// keeps in flight (tracked by vmcnt), and with it for the whole load.  Only
// LDS is ordered here; LDS operations of a wave complete in order.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// Finish this wave's LDS reads and writes, then count one arrival on ctr.
__device__ __forceinline__ void lds_signal(int *ctr) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  if ((threadIdx.x & 63) == 0)
    asm volatile("ds_add_u32 %0, %1" ::"v"(lds_addr(ctr)), "v"(1) : "memory");
}

// Wait until ctr reaches target.  The wait is bounded so that every wave
// exits even if a count were never reached.
__device__ __forceinline__ void lds_wait(const int *ctr, int target) {
  const uint32_t a = lds_addr(ctr);
  for (int it = 0; it < (1 << 18); ++it) {
    int v;
    asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(a) : "memory");
    if (__builtin_amdgcn_readfirstlane(v) >= target)
      break;
    __builtin_amdgcn_s_sleep(1);
  }
}

// Workgroup barrier after this wave's LDS operations have completed.
__device__ __forceinline__ void lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Byte offset of v[row][col] (row < 64 tokens, col < 32 of a state wave's
// columns) in its LDS copy.  The copy is 64-byte slots, one row each, whose
// four 16-byte pieces are permuted: row 16 t + 4 a + b sits in slot
// 16 t + 4 b + a, and its piece p at position p ^ (a & 2).  The reads of the
// substitution's right-hand side (the 16 columns of a tile, rows 4 a + b for
// the four lane groups a) then fall in 32 different banks.
__device__ __forceinline__ int vst_off(int row, int col) {
  const int a = (row >> 2) & 3;
  const int slot = (row & ~15) | ((row & 3) << 2) | a;
  return slot * 64 + 16 * ((col >> 3) ^ (a & 2)) + 2 * (col & 7);
}

} // namespace

// MODE 0: prefill / replay: o, exit states to final_state, checkpoints.
//   Entry states: init[init_idx] (init_idx >= 0), sin[-2 - init_idx]
//   (init_idx <= -2: the planner's scanned entry states), else zero.
// MODE 1: the planner's segment pass: each state wave carries its 32
//   columns of S~ (from 0, values V) and the same 32 columns of M (from the
//   identity, values 0): four column tiles, no o.  S~ leaves to final_state
//   (row-major), M to m_out as hi / lo bf16 at scan_m_bf16_index.  The prep
//   waves build no query operands.
// PRO: the decay gate from logits and the q / k L2 norm run in the prep
// (which of them is decided by A_log != null and qk_eps > 0); EPI: o leaves
// through the output norm and gate.
// One workgroup's work: (chain, head) pair blk of `chains`.
template <int MODE, bool PRO, bool EPI>
__device__ __forceinline__ void fused_body(
    FusedSmem &sm, int blk, const ChainDesc *__restrict__ chains, int32_t H,
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const bf16 *__restrict__ g, const bf16 *__restrict__ beta, bf16 *__restrict__ o,
    const float *__restrict__ init, const float *__restrict__ sin,
    float *__restrict__ final_state, float *__restrict__ m_out, float *__restrict__ ckpt,
    const float *__restrict__ A_log, float g_min, float qk_eps, const bf16 *__restrict__ ogate,
    const float *__restrict__ onw, float oeps) {
  static_assert(MODE == 0 || !EPI, "the segment pass writes no o");
  constexpr bool kQ = MODE == 0; // query operands (Q_decay, M_qk) and o
  constexpr int NC = MODE == 0 ? 2 : 4; // 16-column state tiles per state wave

  const int chain_i = blk / H, h = blk - chain_i * H;
  const ChainDesc cd = chains[chain_i];
  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t rowstride = (int64_t)H * kD;
  const int nch = (cd.ntok + kC - 1) / kC;

  // M_qk blocks (and halves) above the diagonal are zero and never written
  // again; the counters start at 0
  {
    uint32_t *z = reinterpret_cast<uint32_t *>(&sm.a.mqk[0][0]);
    for (int e = tid; e < 8 * 512 / 2; e += kFusedThreads)
      z[e] = 0u;
    if (tid == 0) {
      sm.meet = 0;
      sm.q_done = 0;
      sm.m_done = 0;
      sm.n_ready = 0;
      sm.o_red = 0;
    }
  }
  __syncthreads();

  if (wv < 4) {
    // =========================== state waves ===========================
    const int lane = tid & 63, lr = lane & 15, lg = lane >> 4;
    // columns col0 + 16 (c % 2) + lr of S (MODE 0) or of S~ (c < 2) and M
    // (c >= 2, MODE 1)
    const int col0 = 32 * wv;
    f32x4 S[NC][8]; // rows p = 16 ct + 4 lg + i: channel kperm(p)
    {
      // (each source pointer in a branch of its own: with a select between
      // the two, a kernel holding two inlined bodies crashes the compiler)
      auto load_state = [&](const float *ip) {
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int ct = 0; ct < 8; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              S[c][ct][i] = ip[kperm(16 * ct + 4 * lg + i) * kD + col0 + 16 * c + lr];
      };
      if (MODE == 0 && cd.init_idx >= 0) {
        load_state(init + ((int64_t)cd.init_idx * H + h) * (kD * kD));
      } else if (MODE == 0 && cd.init_idx <= -2) {
        load_state(sin + ((int64_t)(-2 - cd.init_idx) * H + h) * (kD * kD));
      } else {
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
          for (int ct = 0; ct < 8; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int ch = kperm(16 * ct + 4 * lg + i), col = col0 + 16 * (c & 1) + lr;
              S[c][ct][i] = (c >= 2 && ch == col) ? 1.f : 0.f;
            }
      }
    }
    uint8_t *vs = reinterpret_cast<uint8_t *>(&sm.vst[wv][0]);
    // this wave's columns of v for chunk ch, straight into its LDS copy:
    // instruction j, lane l fills slot 16 j + l / 4, position l % 4 (vst_off
    // inverted); rows past the chunk end read 0
    auto load_v = [&](int ch) {
      const int ln = opaque_lane();
      const bool in = ch < nch;
      const int len = in ? min(kC, cd.ntok - ch * kC) : 0;
      const bf16 *vb =
          v + (cd.tok0 + (int64_t)(in ? ch : 0) * kC) * rowstride + (int64_t)h * kD + col0;
      const __amdgpu_buffer_rsrc_t rv =
          buffer_rsrc(vb, in ? (uint32_t)(((len - 1) * rowstride + 32) * 2) : 0u);
      const int piece = (ln & 3) ^ ((ln >> 2) & 2);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = 16 * j + 4 * ((ln >> 2) & 3) + (ln >> 4);
        lds_load16(rv, (int)((row * rowstride + 8 * piece) * 2), vs + 1024 * j);
      }
    };
    load_v(0);
    int ck_next = cd.ckpt_chunk, ck_idx = cd.ckpt_idx;

    for (int step = 0; step <= nch; ++step) {
      if (step > 0) {
        const int ch = step - 1;
        const RecOnce &A = sm.a;
        const RecTwice &B = sm.b[ch & 1];
        const int ln = opaque_lane(), llr = ln & 15, llg = ln >> 4;
        auto frag = [&](const bf16 *blk) { return load_frag(blk + ln * 8); };
        // K_restore^T's A fragment of row tile ct, k-step ks (lane (i, g):
        // channel kperm(16 ct + i), tokens 32 ks + 16 h + 4 g + j at element
        // 4 h + j) from the token-major copy, by two transposed reads: in
        // each 16-lane group, lane 4 a + b of ds_read_b64_tr_b16 receives
        // element b of the 4-element reads of lanes a, a + 4, a + 8, a + 12,
        // so lane L reads token 32 ks + 16 h + 4 g + L / 4 from channel
        // kperm(16 ct + 4 (L % 4)) on (kperm keeps runs of four channels)
        auto kr_frag = [&](const bf16 *kr, int ct, int ks) {
          typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
          const bf16 *p0 =
              kr + (32 * ks + 4 * llg + (llr >> 2)) * kKrLd + kperm(16 * ct + 4 * (llr & 3));
          const bf16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)p0);
          const bf16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(p0 + 16 * kKrLd));
          Frag<bf16> f;
          f.v = __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7);
          return f;
        };
        // W = K_decay S and O^T = S^T Q_decay^T (K = channels; the packed
        // state is the B operand of the first and the A operand of the second),
        // then U by substitution.  MODE 1 runs W, the right-hand side and the
        // substitution for its S~ tiles and then for its M tiles (holding the
        // W of all four at once would exceed the registers).
        [[maybe_unused]] f32x4 Ot[2][4];
        bf16x4 ub[NC][4];
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int hv = 0; hv < NC / 2; ++hv) {
          f32x4 W[2][4];
#pragma unroll
          for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int tt = 0; tt < 4; ++tt)
              W[c][tt] = zero;
          if constexpr (kQ) {
            Frag<bf16> bs[2][4];
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
              for (int s = 0; s < 4; ++s)
                bs[c][s] = pack_acc2(S[c][2 * s], S[c][2 * s + 1]);
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
              for (int tt = 0; tt < 4; ++tt)
                Ot[c][tt] = zero;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              Frag<bf16> ak[4], aq[4];
#pragma unroll
              for (int tt = 0; tt < 4; ++tt) {
                ak[tt] = frag(&A.kd[4 * tt + s][0]);
                aq[tt] = frag(&A.qd[4 * tt + s][0]);
              }
#pragma unroll
              for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                  mma(W[c][tt], ak[tt], bs[c][s]);
                  mma(Ot[c][tt], bs[c][s], aq[tt]);
                }
            }
          } else {
            // the state packed one k-step at a time
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              Frag<bf16> ak[4], bs[2];
#pragma unroll
              for (int tt = 0; tt < 4; ++tt)
                ak[tt] = frag(&A.kd[4 * tt + s][0]);
#pragma unroll
              for (int c = 0; c < 2; ++c)
                bs[c] = pack_acc2(S[2 * hv + c][2 * s], S[2 * hv + c][2 * s + 1]);
#pragma unroll
              for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                for (int c = 0; c < 2; ++c)
                  mma(W[c][tt], ak[tt], bs[c]);
            }
          }
          if (hv == NC / 2 - 1)
            lds_signal(&sm.q_done);
          // Diag(beta) (W - V), the right-hand side of the substitution (M's
          // columns: V = 0); then the next chunk's v into the copy just read
          if (hv == 0)
            wait_vmem_all(); // this chunk's v is in LDS
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) {
            const f32x4 b4 = *reinterpret_cast<const f32x4 *>(&B.beta[16 * tt + 4 * llg]);
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const float vv =
                    hv == 1 ? 0.f
                            : static_cast<float>(*reinterpret_cast<const bf16 *>(
                                  vs + vst_off(16 * tt + 4 * llg + i, 16 * c + llr)));
                W[c][tt][i] = b4[i] * (W[c][tt][i] - vv);
              }
          }
          if (hv == 0) {
            wave_lds_fence();
            load_v(ch + 1);
          }
          // U_I = -D_I^-1 (Diag(beta_I)(W_I - V_I) + sum_{J<I} L_IJ U_J), tile by tile
#pragma unroll
          for (int I = 0; I < 4; ++I) {
            const bf16x4 dn = *reinterpret_cast<const bf16x4 *>(&A.dn[I][ln * 4]);
            bf16x4 lo[3];
#pragma unroll
            for (int J = 0; J < I; ++J)
              lo[J] = *reinterpret_cast<const bf16x4 *>(&A.lo[off_pair(I, J)][ln * 4]);
#pragma unroll
            for (int c = 0; c < 2; ++c) {
              f32x4 a = W[c][I];
#pragma unroll
              for (int J = 0; J < I; ++J)
                a = mma16(a, lo[J], ub[2 * hv + c][J]);
              ub[2 * hv + c][I] = pack4(mma16(zero, dn, pack4(a)));
            }
          }
        }
        // O^T += U^T M_qk^T (K = tokens, kperm order: two stacked U tiles)
        Frag<bf16> bu[NC][2];
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
          for (int s = 0; s < 2; ++s)
            bu[c][s].v = __builtin_shufflevector(ub[c][2 * s], ub[c][2 * s + 1], 0, 1, 2, 3, 4,
                                                 5, 6, 7);
        if constexpr (!kQ)
          lds_signal(&sm.m_done);
        if constexpr (kQ) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          Frag<bf16> am[4];
#pragma unroll
          for (int tt = 0; tt < 4; ++tt)
            am[tt] = frag(&A.mqk[2 * tt + s][0]);
#pragma unroll
          for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int c = 0; c < 2; ++c)
              mma(Ot[c][tt], bu[c][s], am[tt]);
        }
        lds_signal(&sm.m_done);
        {
          // o: lane (lr, lg) holds columns col0 + 16 c + 4 lg .. + 3 of token
          // 16 tt + lr; rows past the chunk end are dropped by the buffer range
          const int len = min(kC, cd.ntok - ch * kC);
          const int64_t tok = cd.tok0 + (int64_t)ch * kC;
          const __amdgpu_buffer_rsrc_t ro =
              buffer_rsrc(o + tok * rowstride + (int64_t)h * kD,
                          (uint32_t)(((len - 1) * rowstride + kD) * 2));
          if constexpr (EPI) {
            // output norm and gate ("Kimi K3.1 Pro 架构完全拆解" §3.3): per
            // token row, o <- sigmoid(gate) w o / sqrt(mean(o^2) + eps); the
            // row's sum of squares is this wave's 32 columns (lane groups
            // combined) plus the other state waves', through LDS
            const __amdgpu_buffer_rsrc_t rgt =
                buffer_rsrc(ogate + tok * rowstride + (int64_t)h * kD,
                            (uint32_t)(((len - 1) * rowstride + kD) * 2));
            u32x2 gz[2][4];
#pragma unroll
            for (int tt = 0; tt < 4; ++tt)
#pragma unroll
              for (int c = 0; c < 2; ++c)
                gz[c][tt] = __builtin_bit_cast(
                    u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                               rgt, (int)(((16 * tt + llr) * rowstride + col0 + 16 * c + 4 * llg) * 2),
                               0, 0));
            float ss[4];
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
              float a = 0.f;
#pragma unroll
              for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                  a += Ot[c][tt][i] * Ot[c][tt][i];
              a = add_xor32(add_xor16(a));
              ss[tt] = a;
            }
            if (llg == 0) {
#pragma unroll
              for (int tt = 0; tt < 4; ++tt)
                sm.ored[wv][16 * tt + llr] = ss[tt];
            }
            lds_signal(&sm.o_red);
            lds_wait(&sm.o_red, 4 * step);
            f32x4 wn[2];
#pragma unroll
            for (int c = 0; c < 2; ++c)
              wn[c] = onw ? *reinterpret_cast<const f32x4 *>(&onw[col0 + 16 * c + 4 * llg])
                          : f32x4{1.f, 1.f, 1.f, 1.f};
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
              const int t = 16 * tt + llr;
              const float rs = __builtin_amdgcn_rsqf(
                  (sm.ored[0][t] + sm.ored[1][t] + sm.ored[2][t] + sm.ored[3][t]) * (1.f / kD) +
                  oeps);
#pragma unroll
              for (int c = 0; c < 2; ++c) {
                float z[4];
                z[0] = __builtin_bit_cast(float, gz[c][tt][0] << 16);
                z[1] = __builtin_bit_cast(float, gz[c][tt][0] & 0xffff0000u);
                z[2] = __builtin_bit_cast(float, gz[c][tt][1] << 16);
                z[3] = __builtin_bit_cast(float, gz[c][tt][1] & 0xffff0000u);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                  Ot[c][tt][i] *= rs * wn[c][i] *
                                  __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-z[i] * kLog2e));
              }
            }
          }
#pragma unroll
          for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int c = 0; c < 2; ++c) {
              const int off =
                  (int)(((16 * tt + llr) * rowstride + col0 + 16 * c + 4 * llg) * 2);
              __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, pack4(Ot[c][tt])),
                                                    ro, off, 0, 0);
            }
        }
        } // kQ
        // S = Diag(a_last) S + K_restore^T U
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
          const f32x4 a4 = *reinterpret_cast<const f32x4 *>(&B.al[16 * ct + 4 * llg]);
#pragma unroll
          for (int c = 0; c < NC; ++c)
            S[c][ct] *= a4;
        }
#pragma unroll
        for (int s = 0; s < 2; ++s) {
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            Frag<bf16> ar[4];
#pragma unroll
            for (int ct = 0; ct < 4; ++ct)
              ar[ct] = kr_frag(&B.kr[0][0], 4 * hf + ct, s);
#pragma unroll
            for (int ct = 0; ct < 4; ++ct)
#pragma unroll
              for (int c = 0; c < NC; ++c)
                mma(S[c][4 * hf + ct], ar[ct], bu[c][s]);
          }
        }
        if (kQ && ckpt != nullptr) {
          if (ch == ck_next && ch <= cd.ckpt_last) {
            float *cp = ckpt + ((int64_t)ck_idx * H + h) * (kD * kD) + col0 + llr;
            ck_next += cd.ckpt_every;
            ++ck_idx;
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
              for (int ct = 0; ct < 8; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                  cp[kperm(16 * ct + 4 * llg + i) * kD + 16 * c] = S[c][ct][i];
          }
        }
      }
      if (step < nch) {
        // -D_w^-1 of the chunk being prepared, in the row layout: the column
        // layout of (I + N^T)^-1 = (I - M)(I + M^2)(I + M^4)(I + M^8) with
        // M = N^T (M_col = N_row, M_row = N_col; mm16_split(c, a_row, b_col)
        // = c + A B in the column layout)
        const int ln = opaque_lane(), llr = ln & 15, llg = ln >> 4;
        lds_wait(&sm.n_ready, 4 * (step + 1));
        const float *N = &sm.ps.nmat[wv][0][0];
        f32x4 Nc;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          Nc[i] = N[(4 * llg + i) * kLdN + llr]; // row 4 lg + i, column lr
        const f32x4 Nr = *reinterpret_cast<const f32x4 *>(&N[llr * kLdN + 4 * llg]);
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        const f32x4 M2c = mm16_split(z, Nc, Nr); // M M
        const f32x4 M2r = mm16_split(z, Nr, Nc); // (M^2)^T = N N
        const f32x4 M4c = mm16_split(z, M2r, M2c);
        const f32x4 M4r = mm16_split(z, M2c, M2r);
        f32x4 eye;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          eye[i] = (4 * llg + i == llr) ? 1.f : 0.f;
        f32x4 Y = mm16_split(eye, M4r, M4c); // I + M^8
        Y = mm16_split(Y, M4r, Y);           // (I + M^4) Y
        Y = mm16_split(Y, M2r, Y);           // (I + M^2) Y
        Y = mm16_split(Y, -Nc, Y);           // (I - M) Y
        // -D_w^-1 as the substitution's A operand (lane (lr, lg): row lr,
        // columns 4 lg .. + 3), once every state wave is done with the
        // previous chunk's
        lds_wait(&sm.m_done, 4 * step);
        *reinterpret_cast<bf16x4 *>(&sm.a.dn[wv][ln * 4]) = pack4(-Y);
        // the next chunk's factor rows of token tile wv, once every tile
        // total is in (the prep waves' meeting): work the prep waves' path,
        // the longer one, would otherwise end with
        lds_wait(&sm.meet, 4 * (step + 2));
        tile_factors(sm.ps, wv, ln);
      }
      lds_sync();
    }
    if (cd.final_idx >= 0) {
      float *fp = final_state + ((int64_t)cd.final_idx * H + h) * (kD * kD) + col0 + lr;
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int ct = 0; ct < 8; ++ct)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            fp[kperm(16 * ct + 4 * lg + i) * kD + 16 * c] = S[c][ct][i];
      if constexpr (MODE == 1) {
        // M as hi / lo bf16 in the planner scan's operand order
        bf16 *fb = reinterpret_cast<bf16 *>(m_out + ((int64_t)cd.final_idx * H + h) * (kD * kD));
#pragma unroll
        for (int c = 2; c < NC; ++c)
#pragma unroll
          for (int ct = 0; ct < 8; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int x = scan_m_bf16_index(kperm(16 * ct + 4 * lg + i), col0 + 16 * (c & 1) + lr);
              const bf16 hi = static_cast<bf16>(S[c][ct][i]);
              fb[x] = hi;
              fb[kD * kD + x] = static_cast<bf16>(S[c][ct][i] - static_cast<float>(hi));
            }
      }
    }
  } else {
    // ============================ prep waves ============================
    // Wave 4 + I, step k: chunk k's decayed operands and tile products, and
    // the tile scan and per-channel factors of chunk k + 1 (so that no
    // exchange of tile totals sits between the start of a step and its
    // elementwise work).
    const int I = wv - 4; // token tile
    u32x4 rg[4], rq[4], rk[4];
    // inputs of chunk ch (an empty range past the last chunk: every load
    // reads 0, and every step issues the same loads)
    auto rsrc_of = [&](const bf16 *base, int ch) {
      const bool in = ch < nch;
      const int len = in ? min(kC, cd.ntok - ch * kC) : 0;
      const int64_t tok = cd.tok0 + (int64_t)(in ? ch : 0) * kC;
      return buffer_rsrc(base + tok * rowstride + (int64_t)h * kD,
                         in ? (uint32_t)(((len - 1) * rowstride + kD) * 2) : 0u);
    };
    // g feeds the tile scan, q and k the elementwise work: each group is
    // loaded right after its previous values are consumed
    auto issue_g = [&](int ch) {
      const int ln = opaque_lane(), llr = ln & 15, llg = ln >> 4;
      const __amdgpu_buffer_rsrc_t r = rsrc_of(g, ch);
#pragma unroll
      for (int s = 0; s < 4; ++s)
        rg[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                              r, (int)(((16 * I + llr) * rowstride + 32 * s +
                                                        8 * llg) * 2), 0, 0));
    };
    // beta of token 16 I + lr of chunk ch, raw bf16 (loaded and stored within
    // one step: a load whose register lives across the step boundary would be
    // waited for there)
    auto load_beta = [&](int ch) -> unsigned short {
      const int ln = opaque_lane(), llr = ln & 15;
      const bool in = ch < nch;
      const int len = in ? min(kC, cd.ntok - ch * kC) : 0;
      const int64_t tok = cd.tok0 + (int64_t)(in ? ch : 0) * kC;
      const __amdgpu_buffer_rsrc_t rbb = buffer_rsrc(
          beta + tok * H + h, in ? (uint32_t)(((len - 1) * (int64_t)H + 1) * 2) : 0u);
      return __builtin_amdgcn_raw_buffer_load_b16(rbb, (int)((16 * I + llr) * H * 2), 0, 0);
    };
    auto store_beta = [&](int ch, unsigned short raw) {
      const int ln = opaque_lane();
      if ((ln >> 4) == 0)
        sm.b[ch & 1].beta[16 * I + (ln & 15)] = __builtin_bit_cast(float, (unsigned)raw << 16);
    };
    auto issue_qk = [&](int ch) {
      const int ln = opaque_lane(), llr = ln & 15, llg = ln >> 4;
      const __amdgpu_buffer_rsrc_t r1 = rsrc_of(k, ch), r2 = rsrc_of(q, ch);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int vo = (int)(((16 * I + llr) * rowstride + 32 * s + 8 * llg) * 2);
        rk[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r1, vo, 0, 0));
        if constexpr (kQ)
          rq[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r2, vo, 0, 0));
      }
    };
    // tile scan of the loaded g (log2 units, inclusive over the 16 tokens of
    // the tile, level by level over all 32 values so that no DPP step waits
    // on the one just issued); lane 15 of each row writes the tile totals
    float G[4][8];
    const bool gate_on = PRO && A_log != nullptr, qk_on = PRO && qk_eps > 0.f;
    // the head's gate scale e^{A_h}, with log2(e) folded into the exponent's
    // scale and into g_min: the gated scan yields log2-unit decays directly
    const float ea = gate_on ? __expf(A_log[h]) : 1.f;
    const float nea2 = -ea * kLog2e, gmin2 = g_min * kLog2e;
    auto scan = [&](int ch) {
      const int ln = opaque_lane(), llr = ln & 15, llg = ln >> 4;
#pragma unroll
      for (int s = 0; s < 4; ++s)
        widen8(rg[s], G[s]);
      if (gate_on) {
        // the log decay from the gate logits, g_min sigmoid(e^{A_h} z), in
        // log2 units; rows past the chunk end decay by nothing
        const bool valid = 16 * I + llr < min(kC, cd.ntok - ch * kC);
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int j = 0; j < 8; ++j)
            G[s][j] = valid ? gmin2 * __builtin_amdgcn_rcpf(
                                          1.f + __builtin_amdgcn_exp2f(G[s][j] * nea2))
                            : 0.f;
      } else {
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int j = 0; j < 8; ++j)
            G[s][j] *= kLog2e;
      }
#pragma unroll
      for (int d = 1; d < 16; d *= 2)
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int j = 0; j < 8; ++j)
            G[s][j] += dpp_shr(G[s][j], d);
      if (llr == 15) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          *reinterpret_cast<f32x4 *>(&sm.ps.tot[I][32 * s + 8 * llg]) =
              f32x4{G[s][0], G[s][1], G[s][2], G[s][3]};
          *reinterpret_cast<f32x4 *>(&sm.ps.tot[I][32 * s + 8 * llg + 4]) =
              f32x4{G[s][4], G[s][5], G[s][6], G[s][7]};
        }
      }
    };
    // the off-diagonal pair (Ip, J): L_IJ = Diag(beta_I) K_loc,I B_IJ^T and
    // M_IJ = Q_loc,I B_IJ^T from the B_IJ fragment blocks and tile Ip's
    // K_loc / Q_loc fragments (lane (lr, lg): row 16 Ip + lr, token
    // 16 J + 4 lg + i)
    auto pair = [&](int Ip, int J, const bf16 *bsrc, const Frag<bf16> (&ak)[4],
                    const Frag<bf16> (&aq)[4], float brow) {
      const int ln = opaque_lane();
      f32x4 accL = {0.f, 0.f, 0.f, 0.f}, accM = accL;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const Frag<bf16> b = load_frag(bsrc + s * 512 + ln * 8);
        mma(accL, b, ak[s]);
        if constexpr (kQ)
          mma(accM, b, aq[s]);
      }
      *reinterpret_cast<bf16x4 *>(&sm.a.lo[off_pair(Ip, J)][ln * 4]) = pack4(accL * brow);
      if constexpr (kQ)
        *reinterpret_cast<bf16x4 *>(&sm.a.mqk[2 * Ip + (J >> 1)][ln * 8 + 4 * (J & 1)]) =
            pack4(accM);
    };

    // chunk 0's beta, tile scan and factors
    issue_g(0);
    issue_qk(0);
    store_beta(0, load_beta(0));
    int meet = 0;
    scan(0);
    issue_g(1);
    meet += 4;
    lds_signal(&sm.meet);
    lds_wait(&sm.meet, meet);
    tile_factors(sm.ps, I, opaque_lane());

    for (int step = 0; step <= nch; ++step) {
      if (step < nch) {
        RecOnce &A = sm.a;
        RecTwice &B = sm.b[step & 1];
        PrepScratch &P = sm.ps;
        const int lane = opaque_lane(), lr = lane & 15, lg = lane >> 4;
        const unsigned short rb_next = load_beta(step + 1);
        if (I == 0) {
          B.al[kperm_inv(2 * lane)] = P.alast[2 * lane];
          B.al[kperm_inv(2 * lane + 1)] = P.alast[2 * lane + 1];
        }
        // ---- elementwise: Q_loc, K_loc, K_st (tile products), Q_decay,
        // K_decay (record, written once the state waves are done with the
        // previous chunk's), K_rs and the scaled pair operands, K_restore
        // (token-major; the state waves read it transposed); the diagonal
        // tile's products ----
        Frag<bf16> fq[4], fk[4], fs[4];
        bf16x8 pq[4], pk[4];
        f32x4 accLc = {0.f, 0.f, 0.f, 0.f}, accMr = accLc;
        float iq = 1.f, ik = 1.f; // 1 / |q|, 1 / |k| of this lane's token
        if (qk_on) {
          // the token's 128 channels sit in lanes lr, lr + 16, lr + 32, lr + 48
          float sq = 0.f, sk = 0.f;
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            if constexpr (kQ)
              sq = sumsq8_bf16(rq[s], sq);
            sk = sumsq8_bf16(rk[s], sk);
          }
          sk = add_xor32(add_xor16(sk));
          ik = __builtin_amdgcn_rsqf(sk + qk_eps);
          if constexpr (kQ) {
            sq = add_xor32(add_xor16(sq));
            iq = __builtin_amdgcn_rsqf(sq + qk_eps);
          }
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          float el[8], es[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            el[j] = __builtin_amdgcn_exp2f(G[s][j]);
            es[j] = __builtin_amdgcn_exp2f(-G[s][j]);
          }
          float fp[8], ft[8], fr[8], qv[8], kv[8];
          load8f(&P.fac[I][0][32 * s + 8 * lg], fp);
          load8f(&P.fac[I][1][32 * s + 8 * lg], ft);
          load8f(&P.fac[I][2][32 * s + 8 * lg], fr);
          if constexpr (kQ) {
            widen8(rq[s], qv);
          } else {
#pragma unroll
            for (int j = 0; j < 8; ++j)
              qv[j] = 0.f;
          }
          widen8(rk[s], kv);
          if (qk_on) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              qv[j] *= iq;
              kv[j] *= ik;
            }
          }
          float xq[8], xk[8], xs[8], yq[8], yk[8], yr[8], yre[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            xq[j] = qv[j] * el[j];  // Q_loc
            xk[j] = kv[j] * el[j];  // K_loc
            xs[j] = kv[j] * es[j];  // K_st
            yq[j] = xq[j] * fp[j];  // Q_decay
            yk[j] = xk[j] * fp[j];  // K_decay
            yr[j] = xs[j] * ft[j];  // K_rs
            yre[j] = yr[j] * fr[j]; // K_restore
          }
          if constexpr (kQ) {
            fq[s] = pack8(xq);
            pq[s] = pack8(yq).v;
          }
          fk[s] = pack8(xk);
          fs[s] = pack8(xs);
          // K_restore into this chunk's token-major copy (the state waves
          // read it transposed)
          *reinterpret_cast<bf16x8 *>(&B.kr[16 * I + lr][32 * s + 8 * lg]) = pack8(yre).v;
          pk[s] = pack8(yk).v;
          // diagonal tile: L_II in the column layout; M_II swapped, in the
          // row layout (row r = lr)
          mma(accLc, fk[s], fs[s]);
          if constexpr (kQ)
            mma(accMr, fs[s], fq[s]);
          if (I < 3)
            *reinterpret_cast<bf16x8 *>(&P.krs[I][s][lane * 8]) = pack8(yr).v;
          if (I == 0) {
            float f3[8], f4[8], b3[8], b4[8];
            load8f(&P.fac[0][3][32 * s + 8 * lg], f3);
            load8f(&P.fac[0][4][32 * s + 8 * lg], f4);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              b3[j] = yr[j] * f3[j];
              b4[j] = yr[j] * f4[j];
            }
            *reinterpret_cast<bf16x8 *>(&P.bsc[0][s][lane * 8]) = pack8(b3).v; // B_20
            *reinterpret_cast<bf16x8 *>(&P.bsc[1][s][lane * 8]) = pack8(b4).v; // B_30
          } else if (I == 1) {
            float f3[8], b3[8];
            load8f(&P.fac[1][3][32 * s + 8 * lg], f3);
#pragma unroll
            for (int j = 0; j < 8; ++j)
              b3[j] = yr[j] * f3[j];
            *reinterpret_cast<bf16x8 *>(&P.bsc[2][s][lane * 8]) = pack8(b3).v; // B_31
          } else if (I == 3) {
            // tile 3's K_loc and Q_loc for the pair (3, 0), which tile 0's wave computes
            *reinterpret_cast<bf16x8 *>(&P.t3k[s][lane * 8]) = fk[s].v;
            if constexpr (kQ)
              *reinterpret_cast<bf16x8 *>(&P.t3q[s][lane * 8]) = fq[s].v;
          }
        }
        // N = strictly lower part of Diag(beta) L_II (lane (lr, lg): row
        // 4 lg + i, column lr), for the state wave that inverts I + N
        {
          const f32x4 bcol = *reinterpret_cast<const f32x4 *>(&B.beta[16 * I + 4 * lg]);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            P.nmat[I][4 * lg + i][lr] = (4 * lg + i > lr) ? bcol[i] * accLc[i] : 0.f;
        }
        lds_signal(&sm.n_ready);
        // (every state wave is done reading the previous chunk's Q_decay, K_decay)
        lds_wait(&sm.q_done, 4 * step);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          if constexpr (kQ)
            *reinterpret_cast<bf16x8 *>(&A.qd[4 * I + s][lane * 8]) = pq[s];
          *reinterpret_cast<bf16x8 *>(&A.kd[4 * I + s][lane * 8]) = pk[s];
        }
        issue_qk(step + 1);
        // next chunk's tile scan (its g was loaded a step ago)
        scan(step + 1);
        issue_g(step + 2);
        // (every state wave is done reading the previous chunk's M_qk, L and,
        // from the other copy, beta)
        lds_wait(&sm.m_done, 4 * step);
        store_beta(step + 1, rb_next);
        if constexpr (kQ) {
          // M_II with its diagonal: rows 16 I + lr, tokens 16 I + 4 lg + i
          f32x4 m = accMr;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            m[i] = (4 * lg + i <= lr) ? m[i] : 0.f;
          *reinterpret_cast<bf16x4 *>(&A.mqk[2 * I + (I >> 1)][lane * 8 + 4 * (I & 1)]) =
              pack4(m);
        }
        meet += 4;
        lds_signal(&sm.meet);
        lds_wait(&sm.meet, meet);

        // ---- off-diagonal tile pairs (B_IJ: K_rs,J itself for J = I - 1,
        // else its scaled copy), two per wave at most ----
        if (I == 0) {
          Frag<bf16> t3k[4], t3q[4];
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            t3k[s] = load_frag(&P.t3k[s][lane * 8]);
            if constexpr (kQ)
              t3q[s] = load_frag(&P.t3q[s][lane * 8]);
          }
          pair(3, 0, &P.bsc[1][0][0], t3k, t3q, B.beta[48 + lr]);
        } else {
          const float brow = B.beta[16 * I + lr];
          if (I == 1) {
            pair(1, 0, &P.krs[0][0][0], fk, fq, brow);
          } else if (I == 2) {
            pair(2, 0, &P.bsc[0][0][0], fk, fq, brow);
            pair(2, 1, &P.krs[1][0][0], fk, fq, brow);
          } else {
            pair(3, 1, &P.bsc[2][0][0], fk, fq, brow);
            pair(3, 2, &P.krs[2][0][0], fk, fq, brow);
          }
        }
      }
      lds_sync();
    }
  }
}

template <int MODE, bool PRO, bool EPI>
__global__ __launch_bounds__(kFusedThreads) void fused_kernel(
    const ChainDesc *__restrict__ chains, int32_t H, const bf16 *__restrict__ q,
    const bf16 *__restrict__ k, const bf16 *__restrict__ v, const bf16 *__restrict__ g,
    const bf16 *__restrict__ beta, bf16 *__restrict__ o, const float *__restrict__ init,
    const float *__restrict__ sin, float *__restrict__ final_state, float *__restrict__ m_out,
    float *__restrict__ ckpt, const float *__restrict__ A_log, float g_min, float qk_eps,
    const bf16 *__restrict__ ogate, const float *__restrict__ onw, float oeps) {
  __shared__ __attribute__((aligned(1024))) FusedSmem sm;
  fused_body<MODE, PRO, EPI>(sm, blockIdx.x, chains, H, q, k, v, g, beta, o, init, sin,
                             final_state, m_out, ckpt, A_log, g_min, qk_eps, ogate, onw, oeps);
}

// The planner's first pass in one launch: the first segment of every split
// sequence from its known entry state (MODE 0: o, and the exit state to
// head_final) in workgroups [0, nhead), the segment pass of the segments
// between its first and last (MODE 1) in the rest.
template <bool PRO, bool EPI>
__global__ __launch_bounds__(kFusedThreads) void fused_pass1_kernel(
    const ChainDesc *__restrict__ heads, int32_t nhead, const ChainDesc *__restrict__ segs,
    int32_t H, const bf16 *__restrict__ q, const bf16 *__restrict__ k,
    const bf16 *__restrict__ v, const bf16 *__restrict__ g, const bf16 *__restrict__ beta,
    bf16 *__restrict__ o, const float *__restrict__ init, float *__restrict__ head_final,
    float *__restrict__ ckpt, float *__restrict__ st_out, float *__restrict__ m_out,
    const float *__restrict__ A_log, float g_min, float qk_eps, const bf16 *__restrict__ ogate,
    const float *__restrict__ onw, float oeps) {
  __shared__ __attribute__((aligned(1024))) FusedSmem sm;
  const int b = blockIdx.x;
  if (b < nhead)
    fused_body<0, PRO, EPI>(sm, b, heads, H, q, k, v, g, beta, o, init, nullptr, head_final,
                            nullptr, ckpt, A_log, g_min, qk_eps, ogate, onw, oeps);
  else
    fused_body<1, PRO, false>(sm, b - nhead, segs, H, q, k, v, g, beta, nullptr, nullptr,
                              nullptr, st_out, m_out, nullptr, A_log, g_min, qk_eps, nullptr,
                              nullptr, 0.f);
}

hipError_t launch_fused_pass1(const ChainDesc *heads, int32_t nheads, const ChainDesc *segs,
                              int32_t nsegs, int32_t H, const void *q, const void *k,
                              const void *v, const void *g, const void *beta, void *o,
                              const float *init, float *head_final, float *ckpt, float *st_out,
                              float *m_out, hipStream_t s, const Prologue &pro,
                              const Epilogue &epi) {
  const int64_t nb = ((int64_t)nheads + nsegs) * H;
  if (nb == 0)
    return hipSuccess;
  dim3 grid((unsigned)nb), block(kFusedThreads);
  const int32_t nhead = nheads * H;
  auto launch = [&](auto kern) {
    kern<<<grid, block, 0, s>>>(heads, nhead, segs, H, (const bf16 *)q, (const bf16 *)k,
                                (const bf16 *)v, (const bf16 *)g, (const bf16 *)beta, (bf16 *)o,
                                init, head_final, ckpt, st_out, m_out, pro.A_log, pro.g_min,
                                pro.qk_eps, (const bf16 *)epi.gate, epi.weight, epi.eps);
  };
  if (epi.on())
    launch(fused_pass1_kernel<true, true>);
  else if (pro.on())
    launch(fused_pass1_kernel<true, false>);
  else
    launch(fused_pass1_kernel<false, false>);
  return hipGetLastError();
}

hipError_t launch_fused(const ChainDesc *chains, int32_t nchains, int32_t H, const void *q,
                         const void *k, const void *v, const void *g, const void *beta,
                         void *o, const float *init, const float *sin, float *final_state,
                         float *ckpt, hipStream_t s, const Prologue &pro, const Epilogue &epi) {
  if (nchains == 0)
    return hipSuccess;
  dim3 grid((unsigned)((int64_t)nchains * H)), block(kFusedThreads);
  auto launch = [&](auto kern) {
    kern<<<grid, block, 0, s>>>(chains, H, (const bf16 *)q, (const bf16 *)k, (const bf16 *)v,
                                (const bf16 *)g, (const bf16 *)beta, (bf16 *)o, init, sin,
                                final_state, nullptr, ckpt, pro.A_log, pro.g_min, pro.qk_eps,
                                (const bf16 *)epi.gate, epi.weight, epi.eps);
  };
  if (epi.on())
    launch(fused_kernel<0, true, true>);
  else if (pro.on())
    launch(fused_kernel<0, true, false>);
  else
    launch(fused_kernel<0, false, false>);
  return hipGetLastError();
}

} // namespace kda
