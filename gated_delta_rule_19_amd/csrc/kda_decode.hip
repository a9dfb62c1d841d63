// KDA decode step: one token per sequence, fp32 state updated in place.
//
// Follows the alternative ("u") form of the recurrence that the pages'
// decode kernel follows ("Kimi K3 的架構" (hao.cnyes.com), §六 FlashKDA 演算法;
// cost model in its 複雜度分析 part: about 7 D^2 FLOPs and 8 D^2 bytes of
// fp32 state traffic per head per token):
//     DS = Diag(exp g) S,  w = DS^T k,  y = DS^T q,
//     u  = beta (v - w),   S' = DS + k u^T,   o = S'^T q = y + (k . q) u.
//
// The kernel is HBM-bound.  One 256-thread workgroup owns one (sequence,
// head) state of 128 x 128 fp32 (64 KiB).  Thread t holds rows
// 16*(t/32) .. +15 of the four columns 4*(t%32) .. +3 in registers, so the
// state is read once and written once, with each wave touching two full
// 512-byte rows per instruction.  Both reductions (DS^T k and DS^T q) come out
// of the same pass; the column sums cross the eight row groups through LDS.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

// The layer's steps around the recurrence, for the LAYER variants of the
// kernels below ("Kimi K3.1 Pro 架构完全拆解" §3.2, §3.3, §3.4: the decode /
// replay kernel also does the input normalization, the gating and the output
// norm).  The norms act as scalars: with ik = 1/|k| and iq = 1/|q|,
//   w = ik (DS^T k),  y = iq (DS^T q),  k.q -> ik iq (k.q),  S' = DS + k (ik u)^T,
// so the raw k and q stay in LDS.  The output norm takes the 128 outputs of
// a (sequence, head) row, which are this workgroup's.
template <typename T> struct LayerArgs {
  const float *A_log;  // [H] or null: g holds the log decay itself
  float g_min;
  float qk_eps;        // > 0: q, k normalized
  const T *ogate;      // output gate logits (laid out like o), or null
  const float *onw;    // [dv] or null
  float oeps;
};

// Wave 0: k.q, and (LAYER) the inverse norms; results to LDS.
template <bool LAYER, typename T>
__device__ __forceinline__ void kq_norms(int tid, const float *s_k, const float *s_q,
                                         const LayerArgs<T> &la, float *s_kq, float *s_ik,
                                         float *s_iq) {
  if (tid < 64) {
    float p = s_k[tid] * s_q[tid] + s_k[tid + 64] * s_q[tid + 64];
    float pk = 0.f, pq = 0.f;
    const bool qk = LAYER && la.qk_eps > 0.f;
    if (qk) {
      pk = s_k[tid] * s_k[tid] + s_k[tid + 64] * s_k[tid + 64];
      pq = s_q[tid] * s_q[tid] + s_q[tid + 64] * s_q[tid + 64];
    }
    p = add_xor16(add_xor32(p));
    if (qk) {
      pk = add_xor16(add_xor32(pk));
      pq = add_xor16(add_xor32(pq));
    }
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) {
      p += __shfl_xor(p, m);
      if (qk) {
        pk += __shfl_xor(pk, m);
        pq += __shfl_xor(pq, m);
      }
    }
    if (tid == 0) {
      const float ik = qk ? __builtin_amdgcn_rsqf(pk + la.qk_eps) : 1.f;
      const float iq = qk ? __builtin_amdgcn_rsqf(pq + la.qk_eps) : 1.f;
      *s_kq = p * ik * iq;
      *s_ik = ik;
      *s_iq = iq;
    }
  }
}

// Threads 0..127 (two whole waves) hold one output each: its RMS norm over
// the 128 and the gate.  Call once with `store` false before a barrier (the
// per-wave sums of squares go to s_ss), then with `store` true after it.
__device__ __forceinline__ float out_norm_sum(int tid, float x, float *s_ss) {
  float p = add_xor16(add_xor32(x * x));
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1)
    p += __shfl_xor(p, m);
  if ((tid & 63) == 0)
    s_ss[tid >> 6] = p;
  return x;
}
__device__ __forceinline__ float out_norm_apply(int tid, float x, float z, const float *s_ss,
                                                const float *onw, float eps) {
  const float sc = __builtin_amdgcn_rsqf((s_ss[0] + s_ss[1]) * (1.f / kD) + eps);
  const float sg = __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-z * 1.4426950408889634f));
  return x * sc * (onw ? onw[tid] : 1.f) * sg;
}

template <typename T, bool LAYER>
__global__ __launch_bounds__(256) void decode_kernel(const T *__restrict__ q,
                                                     const T *__restrict__ k,
                                                     const T *__restrict__ v,
                                                     const T *__restrict__ g,
                                                     const T *__restrict__ beta,
                                                     float *__restrict__ state,
                                                     T *__restrict__ o, int32_t H,
                                                     LayerArgs<T> la) {
  const int64_t nh = blockIdx.x;
  const int tid = threadIdx.x;
  const int cg = tid & 31; // column group: columns 4*cg .. 4*cg+3
  const int rg = tid >> 5; // row group: rows 16*rg .. 16*rg+15

  __shared__ float s_k[kD], s_q[kD], s_a[kD], s_v[kD], s_u[kD];
  __shared__ float s_w[8][kD], s_y[8][kD];
  __shared__ float s_kq, s_beta, s_ik, s_iq, s_ss[2];

  float *S = state + nh * (int64_t)(kD * kD);
  f32x4 s[16];
#pragma unroll
  for (int i = 0; i < 16; ++i)
    s[i] = __builtin_nontemporal_load(
        reinterpret_cast<const f32x4 *>(S + (16 * rg + i) * kD + 4 * cg));

  const bool epi = LAYER && la.ogate != nullptr;
  float zo = 0.f; // this thread's output gate logit (tid < 128)
  if (tid < kD) {
    const int64_t off = nh * kD + tid;
    s_k[tid] = to_f32(k[off]);
    s_q[tid] = to_f32(q[off]);
    float gg = to_f32(g[off]);
    if (LAYER && la.A_log)
      gg = gate_log_decay(gg, __expf(la.A_log[nh % H]), la.g_min);
    s_a[tid] = __expf(gg);
    s_v[tid] = to_f32(v[off]);
    if (epi)
      zo = to_f32(la.ogate[off]);
  }
  if (tid == 0)
    s_beta = to_f32(beta[nh]);
  __syncthreads();

  // k . q (and the inverse norms), reduced inside wave 0
  kq_norms<LAYER>(tid, s_k, s_q, la, &s_kq, &s_ik, &s_iq);

  f32x4 w = {0.f, 0.f, 0.f, 0.f}, y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = 16 * rg + i;
    s[i] *= s_a[r];
    w += s_k[r] * s[i];
    y += s_q[r] * s[i];
  }
  *reinterpret_cast<f32x4 *>(&s_w[rg][4 * cg]) = w;
  *reinterpret_cast<f32x4 *>(&s_y[rg][4 * cg]) = y;
  __syncthreads();

  float ov = 0.f;
  if (tid < kD) {
    float ws = 0.f, ys = 0.f;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      ws += s_w[r][tid];
      ys += s_y[r][tid];
    }
    const float ik = LAYER ? s_ik : 1.f, iq = LAYER ? s_iq : 1.f;
    const float u = s_beta * (s_v[tid] - ik * ws);
    s_u[tid] = ik * u;
    ov = iq * ys + s_kq * u;
    if (epi)
      out_norm_sum(tid, ov, s_ss);
    else
      o[nh * kD + tid] = from_f32<T>(ov);
  }
  __syncthreads();
  if (epi && tid < kD)
    o[nh * kD + tid] = from_f32<T>(out_norm_apply(tid, ov, zo, s_ss, la.onw, la.oeps));

  const f32x4 u4 = *reinterpret_cast<const f32x4 *>(&s_u[4 * cg]);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = 16 * rg + i;
    const f32x4 nv = s[i] + s_k[r] * u4;
    __builtin_nontemporal_store(nv, reinterpret_cast<f32x4 *>(S + r * kD + 4 * cg));
  }
}

// Speculative-decode replay ("Kimi K3.1 Pro 架构完全拆解" §3.4; "部署 Kimi K3：
// 从 KDA Kernel 到 Fleet 调度" §四): instead of restoring a state snapshot,
// the state before a draft window is advanced through the m accepted draft
// tokens from their cached projected inputs, then through the P new tokens
// (the bonus token first, then the next window's drafts), all on chip.  The
// state after the bonus token is written back; the new tokens' outputs are
// written; the later drafts' states are not kept.  The layout and the step
// are the decode kernel's: the state is read once and written once however
// many tokens the call runs.
template <typename T, bool LAYER>
__global__ __launch_bounds__(256) void replay_kernel(
    int32_t H, int32_t W, int32_t P, const int32_t *__restrict__ accepted,
    const T *__restrict__ ck, const T *__restrict__ cv, const T *__restrict__ cg,
    const T *__restrict__ cb, const T *__restrict__ q, const T *__restrict__ k,
    const T *__restrict__ v, const T *__restrict__ g, const T *__restrict__ beta,
    float *__restrict__ state, T *__restrict__ o, LayerArgs<T> la) {
  const int64_t nh = blockIdx.x;
  const int n = (int)(nh / H), h = (int)(nh - (int64_t)n * H);
  const int tid = threadIdx.x;
  const int cg4 = tid & 31; // column group: columns 4*cg4 .. 4*cg4+3
  const int rg = tid >> 5;  // row group: rows 16*rg .. 16*rg+15

  __shared__ float s_k[kD], s_q[kD], s_a[kD], s_v[kD], s_u[kD];
  __shared__ float s_w[8][kD], s_y[8][kD];
  __shared__ float s_kq, s_beta, s_ik, s_iq, s_ss[2];

  float *S = state + nh * (int64_t)(kD * kD);
  f32x4 s[16];
#pragma unroll
  for (int i = 0; i < 16; ++i)
    s[i] = __builtin_nontemporal_load(
        reinterpret_cast<const f32x4 *>(S + (16 * rg + i) * kD + 4 * cg4));
  // the layer's steps apply to cached and new tokens alike (per token,
  // elementwise or per row), so the cache may hold the raw inputs
  const bool epi = LAYER && la.ogate != nullptr;
  const float ea = (LAYER && la.A_log) ? __expf(la.A_log[h]) : 1.f;

  const int m = min(max(accepted[n], 0), W); // accepted draft tokens to replay
  const int total = m + P;
  const int commit = m + min(P, 1); // tokens whose state is kept
  // one token's inputs for thread tid < 128 (element tid of k, g, v, q) and
  // beta; the next token's are loaded while the current one is stepped
  struct TokIn {
    float k, g, v, q, b, z;
  };
  auto load_tok = [&](int t) {
    TokIn x = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (t >= total)
      return x;
    const bool out = t >= m;
    const int64_t tok = out ? ((int64_t)n * P + (t - m)) * H + h : ((int64_t)n * W + t) * H + h;
    if (tid < kD) {
      x.k = to_f32((out ? k : ck)[tok * kD + tid]);
      x.g = to_f32((out ? g : cg)[tok * kD + tid]);
      x.v = to_f32((out ? v : cv)[tok * kD + tid]);
      if (out) // (q may be null when P = 0)
        x.q = to_f32(q[tok * kD + tid]);
      if (out && epi)
        x.z = to_f32(la.ogate[tok * kD + tid]);
    }
    if (tid == 0)
      x.b = to_f32((out ? beta : cb)[tok]);
    return x;
  };
  TokIn cur = load_tok(0);
  for (int t = 0; t < total; ++t) {
    const bool out = t >= m; // a new token: its output is written
    const int64_t tok = out ? ((int64_t)n * P + (t - m)) * H + h : 0;
    if (tid < kD) {
      s_k[tid] = cur.k;
      s_a[tid] = __expf((LAYER && la.A_log) ? gate_log_decay(cur.g, ea, la.g_min) : cur.g);
      s_v[tid] = cur.v;
      s_q[tid] = cur.q;
    }
    if (tid == 0)
      s_beta = cur.b;
    const TokIn nxt = load_tok(t + 1);
    __syncthreads();

    // k . q (and the inverse norms), inside wave 0
    kq_norms<LAYER>(tid, s_k, s_q, la, &s_kq, &s_ik, &s_iq);
    f32x4 w = {0.f, 0.f, 0.f, 0.f}, y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = 16 * rg + i;
      s[i] *= s_a[r];
      w += s_k[r] * s[i];
      y += s_q[r] * s[i];
    }
    *reinterpret_cast<f32x4 *>(&s_w[rg][4 * cg4]) = w;
    *reinterpret_cast<f32x4 *>(&s_y[rg][4 * cg4]) = y;
    __syncthreads();

    float ov = 0.f;
    if (tid < kD) {
      float ws = 0.f, ys = 0.f;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        ws += s_w[r][tid];
        ys += s_y[r][tid];
      }
      const float ik = LAYER ? s_ik : 1.f, iq = LAYER ? s_iq : 1.f;
      const float u = s_beta * (s_v[tid] - ik * ws);
      s_u[tid] = ik * u;
      ov = iq * ys + s_kq * u;
      if (out && epi)
        out_norm_sum(tid, ov, s_ss);
      else if (out)
        o[tok * kD + tid] = from_f32<T>(ov);
    }
    __syncthreads();
    if (out && epi && tid < kD)
      o[tok * kD + tid] = from_f32<T>(out_norm_apply(tid, ov, cur.z, s_ss, la.onw, la.oeps));

    const f32x4 u4 = *reinterpret_cast<const f32x4 *>(&s_u[4 * cg4]);
#pragma unroll
    for (int i = 0; i < 16; ++i)
      s[i] += s_k[16 * rg + i] * u4;
    if (t + 1 == commit) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        __builtin_nontemporal_store(
            s[i], reinterpret_cast<f32x4 *>(S + (16 * rg + i) * kD + 4 * cg4));
    }
    cur = nxt;
    __syncthreads(); // the next token rewrites the shared inputs
  }
}

template <typename T> static LayerArgs<T> layer_args(const Epilogue &epi, const Prologue &pro) {
  return LayerArgs<T>{pro.A_log, pro.g_min, pro.qk_eps, (const T *)epi.gate, epi.weight, epi.eps};
}

hipError_t launch_replay(int elt, int32_t N, int32_t H, int32_t W, const int32_t *accepted,
                         const void *ck, const void *cv, const void *cg, const void *cb,
                         int32_t P, const void *q, const void *k, const void *v, const void *g,
                         const void *beta, float *state, void *o, const Prologue &pro,
                         const Epilogue &epi, hipStream_t s) {
  const int64_t nh = (int64_t)N * H;
  if (nh == 0)
    return hipSuccess;
  dim3 grid((unsigned)nh), block(256);
  const bool layer = pro.on() || epi.on();
  auto run = [&](auto kern, auto tag) {
    using T = decltype(tag);
    kern<<<grid, block, 0, s>>>(H, W, P, accepted, (const T *)ck, (const T *)cv, (const T *)cg,
                                (const T *)cb, (const T *)q, (const T *)k, (const T *)v,
                                (const T *)g, (const T *)beta, state, (T *)o,
                                layer_args<T>(epi, pro));
  };
  if (elt == 1)
    layer ? run(replay_kernel<bf16, true>, bf16()) : run(replay_kernel<bf16, false>, bf16());
  else
    layer ? run(replay_kernel<float, true>, 0.f) : run(replay_kernel<float, false>, 0.f);
  return hipGetLastError();
}

hipError_t launch_decode(int elt, int32_t N, int32_t H, const void *q, const void *k,
                         const void *v, const void *g, const void *beta, float *state, void *o,
                         const Prologue &pro, const Epilogue &epi, hipStream_t s) {
  const int64_t nh = (int64_t)N * H;
  if (nh == 0)
    return hipSuccess;
  dim3 grid((unsigned)nh), block(256);
  const bool layer = pro.on() || epi.on();
  auto run = [&](auto kern, auto tag) {
    using T = decltype(tag);
    kern<<<grid, block, 0, s>>>((const T *)q, (const T *)k, (const T *)v, (const T *)g,
                                (const T *)beta, state, (T *)o, H, layer_args<T>(epi, pro));
  };
  if (elt == 1)
    layer ? run(decode_kernel<bf16, true>, bf16()) : run(decode_kernel<bf16, false>, bf16());
  else
    layer ? run(decode_kernel<float, true>, 0.f) : run(decode_kernel<float, false>, 0.f);
  return hipGetLastError();
}

} // namespace kda
