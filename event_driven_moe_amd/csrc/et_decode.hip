// et_decode.hip -- one decode step's attention front as one persistent kernel.
//
// Event Tensor notes, section "端到端低 batch serving": the megakernel covers
// the decoding pipeline, and the query branch's Norm + RoPE runs in parallel
// with the key branch's Norm + RoPE + cache append.  Task kinds, for
// sequence b and key/value head h (i = b * Hk + h):
//   query branch  (b, h): RMSNorm + RoPE of the G = Hq / Hk query heads that
//                 read key/value head h -> rotated queries (fp32, workspace);
//   key branch    (b, h): RMSNorm + RoPE of key head h -> appended to the key
//                 cache at position pos[b] (bf16); the value row appended to
//                 the value cache;
//   attention split (b, h, j): waits on E_qk[i] (wait count 2: one notify
//                 from each branch), then the online softmax of the G query
//                 heads over its share of positions 0 .. pos[b] (split j of NS
//                 equal ranges of the cache, chunks of 256 positions): running
//                 max, sum and unnormalised output to the workspace; notifies
//                 E_att[i] (wait count NS);
//   merge         (b, h): after E_att[i], out = sum_j e^(m_j - M) o_j /
//                 sum_j e^(m_j - M) l_j with M = max_j m_j.
// Splitting the positions puts NS workgroups on each (sequence, head): at a
// batch of one sequence the attention is a chain of memory latencies, and a
// single workgroup per head walked 600 positions in 110 us.
// Static and dynamic schedules interleave the two branches' tasks (ids 2i,
// 2i + 1), so they run at the same time on different compute units; the
// barrier baseline runs them as two operators with a global event between
// them, and the per-operator baseline as three launches.
#include "et_device.hpp"
#include "et_launch.hpp"

namespace et {

struct DecodeArgs {
  const uint16_t* q;    // [B, Hq, D] bf16
  const uint16_t* k;    // [B, Hk, D]
  const uint16_t* v;    // [B, Hk, D]
  const uint16_t* wq;   // [D] query-norm weight
  const uint16_t* wk;   // [D] key-norm weight
  const int* pos;       // [B] position of each sequence's new token
  uint16_t* kc;         // [B, S, Hk, D] key cache
  uint16_t* vc;         // [B, S, Hk, D] value cache
  float* qr;            // [B, Hq, D] rotated queries (workspace)
  float* po;            // [B * Hk, NS, G, D] split partial outputs (workspace)
  float* pml;           // [B * Hk, NS, G, 2] split running max and sum (workspace)
  float* out;           // [B, Hq, D]
  int B, Hq, Hk, S, G;
  int NS, L;            // attention splits per (sequence, head), positions per split
  float theta_log2;     // log2 of the RoPE base
  float eps;
  int ev_qk;            // E_qk[b * Hk + h]
  int ev_att;           // E_att[b * Hk + h]
};

constexpr int kHeadDim = 128;         // D: lane l holds elements l and l + 64
constexpr int kMaxGroup = 16;         // G = Hq / Hk
constexpr int kAttnChunk = kThreads;  // positions per online-softmax chunk
constexpr int kMaxSplits = 8;         // attention splits per (sequence, head)
enum : int { EV_QALL = 0, EV_KALL = 1, EV_ATT = 2, EV_DEC_FIXED = 8 };

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// RMSNorm over one head (lane l: elements l and l + 64), then the rotation of
// the pair (l, l + 64) by pos * theta^(-2l/D).
__device__ __forceinline__ void norm_rope(float& x0, float& x1, const uint16_t* w, int pos,
                                          const DecodeArgs& a) {
  const int l = threadIdx.x & 63;
  const float ss = wave_sum(x0 * x0 + x1 * x1);
  const float r = 1.0f / __builtin_sqrtf(ss * (1.0f / kHeadDim) + a.eps);
  const float y0 = x0 * r * bf16_to_f32(w[l]);
  const float y1 = x1 * r * bf16_to_f32(w[l + 64]);
  const float inv = exp2f(-(float)(2 * l) * (1.0f / kHeadDim) * a.theta_log2);
  float sn, cs;
  sincosf((float)pos * inv, &sn, &cs);
  x0 = y0 * cs - y1 * sn;
  x1 = y1 * cs + y0 * sn;
}

// GM: the largest group G = Hq / Hk the instance handles (8 or 16); the
// value accumulators of a lane take 8 * GM registers.
template <int GM>
__global__ __launch_bounds__(kThreads, 1) void decode_kernel(RunArgs ra, DecodeArgs a) {
  __shared__ Shared sh;
  __shared__ __align__(16) float qs[GM][kHeadDim];
  __shared__ __align__(16) float sc[GM][kAttnChunk];
  __shared__ __align__(16) float part[4][GM][kHeadDim];
  __shared__ float m_run[GM], l_run[GM], alpha[GM];

  Ctx c;
  if (!prologue(c, ra, &sh)) return;
  const int sched = ra.sched;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int N = a.B * a.Hk;
  const bool interleaved = sched == ET_SCHED_STATIC || sched == ET_SCHED_DYNAMIC;
  const int G = a.G;

  auto seq_pos = [&](int b, int task) ET_INLINE -> int {
    const int p = a.pos[b];
    if (p < 0 || p >= a.S) {
      if (tid == 0) raise_fault(ra, ET_ERANGE, task, b, p);
      return -1;
    }
    return p;
  };

  // both branches notify E_qk[i]; the second one fires it (dynamic: it
  // pushes the attention splits of (b, h))
  auto branch_done = [&](int i, int task, int op_event) ET_INLINE {
    if (sched == ET_SCHED_PER_OP) return;
    wg_release();
    if (sched == ET_SCHED_BARRIER) {
      t0_notify_bcast(c, op_event, op_event, 1, N, task);
    } else if (sched == ET_SCHED_STATIC) {
      t0_notify(c, a.ev_qk + i, 1, 2, task);
    } else if (wg_notify(c, a.ev_qk + i, 1, 2, task)) {
      wg_push(c, a.NS, [&](int j) { return 2 * N + i * a.NS + j; },
              [&](int j) { return i * a.NS + j; });
    }
  };

  auto query_branch = [&](int i, int task) ET_INLINE -> bool {
    const int b = i / a.Hk, h = i % a.Hk;
    const int p = seq_pos(b, task);
    if (p < 0) return false;
    for (int g = wave; g < G; g += 4) {
      const size_t row = ((size_t)b * a.Hq + h * G + g) * kHeadDim;
      float x0 = bf16_to_f32(a.q[row + lane]), x1 = bf16_to_f32(a.q[row + lane + 64]);
      norm_rope(x0, x1, a.wq, p, a);
      st_coh(&a.qr[row + lane], x0);
      st_coh(&a.qr[row + lane + 64], x1);
    }
    branch_done(i, task, EV_QALL);
    return true;
  };

  auto key_branch = [&](int i, int task) ET_INLINE -> bool {
    const int b = i / a.Hk, h = i % a.Hk;
    if (sched == ET_SCHED_BARRIER && !wg_wait_bcast(c, EV_QALL, EV_QALL, task)) return false;
    const int p = seq_pos(b, task);
    if (p < 0) return false;
    if (wave == 0) {
      const size_t src = ((size_t)b * a.Hk + h) * kHeadDim;
      const size_t dst = (((size_t)b * a.S + p) * a.Hk + h) * kHeadDim;
      float x0 = bf16_to_f32(a.k[src + lane]), x1 = bf16_to_f32(a.k[src + lane + 64]);
      norm_rope(x0, x1, a.wk, p, a);
      st_coh(&a.kc[dst + lane], f32_to_bf16(x0));
      st_coh(&a.kc[dst + lane + 64], f32_to_bf16(x1));
      st_coh(&a.vc[dst + lane], a.v[src + lane]);
      st_coh(&a.vc[dst + lane + 64], a.v[src + lane + 64]);
    }
    branch_done(i, task, EV_KALL);
    return true;
  };

  auto attention = [&](int i, int split, int task) ET_INLINE -> bool {
    const int b = i / a.Hk, h = i % a.Hk;
    if (sched == ET_SCHED_STATIC) {
      if (!wg_wait(c, a.ev_qk + i, 2, task)) return false;
    } else if (sched == ET_SCHED_BARRIER) {
      if (!wg_wait_bcast(c, EV_KALL, EV_KALL, task)) return false;
    }
    const int p = seq_pos(b, task);
    if (p < 0) return false;
    const int n = p + 1;
    const int p0 = split * a.L, p1 = min(n, p0 + a.L);   // this split's positions
    const float scale = 1.0f / __builtin_sqrtf((float)kHeadDim);
    const size_t q0 = ((size_t)b * a.Hq + h * G) * kHeadDim;
    for (int x = tid; x < G * kHeadDim; x += kThreads) qs[x / kHeadDim][x % kHeadDim] = ld_coh(&a.qr[q0 + x]);
    if (tid < G) {
      m_run[tid] = -__builtin_inff();
      l_run[tid] = 0.f;
    }
    __syncthreads();
    const size_t rstride = (size_t)a.Hk * kHeadDim;                 // elements between positions
    const size_t base = ((size_t)b * a.S * a.Hk + h) * kHeadDim;    // position 0 of this head
    const Rsrc rk = make_rsrc(a.kc + base, (uint32_t)((size_t)n * rstride * 2));
    // value rows: lane (rq = lane / 16, cc = lane % 16) accumulates columns
    // 8 cc .. 8 cc + 7 of the rows 4 r + rq its wave takes
    const int rq = lane >> 4, cc = lane & 15;
    float o[GM][8];
#pragma unroll
    for (int g = 0; g < GM; ++g)
#pragma unroll
      for (int j = 0; j < 8; ++j) o[g][j] = 0.f;
    // The newest position (n - 1) was written in this launch and is read
    // with coherent loads; the others are inputs.  A chunk's key rows are
    // requested before the previous chunk's value rows are used, and each
    // wave requests its value rows of a chunk in one or two batches of
    // 16-byte loads (a 4-byte load per lane per row, 16 rows in flight per
    // wave, put about five memory latencies on every chunk).
    const int qlast = n - 1;
    const Rsrc rv = make_rsrc(a.vc + base, (uint32_t)((size_t)n * rstride * 2));
    i32x4 kr[kHeadDim / 8];
    auto load_keys = [&](int c0) ET_INLINE {
      const int pp = c0 + tid;
      const uint32_t off = pp < p1 ? (uint32_t)(pp * rstride * 2) : kOOB;
      if (pp == qlast) {
#pragma unroll
        for (int j = 0; j < kHeadDim / 8; ++j) kr[j] = ld16c(rk, off + 16u * j);
      } else {
#pragma unroll
        for (int j = 0; j < kHeadDim / 8; ++j) kr[j] = ld16(rk, off + 16u * j);
      }
    };
    constexpr int kVB = GM <= 8 ? 16 : 8;      // value loads per batch per lane
    if (p0 < p1) load_keys(p0);
    for (int c0 = p0; c0 < p1; c0 += kAttnChunk) {
      // scores of position c0 + tid for every head of the group
      const int pp = c0 + tid;
      float s[GM];
#pragma unroll
      for (int g = 0; g < GM; ++g) s[g] = 0.f;
#pragma unroll
      for (int j = 0; j < kHeadDim / 8; ++j) {
        float kf[8];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          kf[2 * t] = __builtin_bit_cast(float, (uint32_t)kr[j][t] << 16);
          kf[2 * t + 1] = __builtin_bit_cast(float, (uint32_t)kr[j][t] & 0xffff0000u);
        }
#pragma unroll
        for (int g = 0; g < GM; ++g)
          if (g < G) {
            const float4 qa = *reinterpret_cast<const float4*>(&qs[g][8 * j]);
            const float4 qb = *reinterpret_cast<const float4*>(&qs[g][8 * j + 4]);
            s[g] += qa.x * kf[0] + qa.y * kf[1] + qa.z * kf[2] + qa.w * kf[3] +
                    qb.x * kf[4] + qb.y * kf[5] + qb.z * kf[6] + qb.w * kf[7];
          }
      }
      for (int g = 0; g < G; ++g) sc[g][tid] = pp < p1 ? s[g] * scale : -__builtin_inff();
      __syncthreads();
      // online softmax: wave w updates the running max and sum of heads w, w+4, ...
      for (int g = wave; g < G; g += 4) {
        float mx = fmaxf(fmaxf(sc[g][lane], sc[g][lane + 64]), fmaxf(sc[g][lane + 128], sc[g][lane + 192]));
        mx = wave_max(mx);
        const float mnew = fmaxf(m_run[g], mx);
        float sum = 0.f;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float e = __expf(sc[g][lane + 64 * u] - mnew);
          sc[g][lane + 64 * u] = e;
          sum += e;
        }
        sum = wave_sum(sum);
        if (lane == 0) {
          const float al = __expf(m_run[g] - mnew);
          alpha[g] = al;
          l_run[g] = l_run[g] * al + sum;
          m_run[g] = mnew;
        }
      }
      __syncthreads();
#pragma unroll
      for (int g = 0; g < GM; ++g)
        if (g < G) {
          const float al = alpha[g];
#pragma unroll
          for (int j = 0; j < 8; ++j) o[g][j] *= al;
        }
      // rows past the split's end load nothing and carry probability 0
      const int cend = min(p1, c0 + kAttnChunk);
      const bool coh = qlast >= c0 && qlast < cend;
#pragma unroll
      for (int t0 = 0; t0 < 16; t0 += kVB) {
        i32x4 vv[kVB];
#pragma unroll
        for (int t = 0; t < kVB; ++t) {
          const int q = c0 + 16 * (t0 + t) + 4 * wave + rq;
          const uint32_t off = q < cend ? (uint32_t)((q * rstride + 8 * cc) * 2) : kOOB;
          vv[t] = coh ? ld16c(rv, off) : ld16(rv, off);
        }
        // the next chunk's key rows, behind this chunk's value rows
        if (t0 + kVB == 16 && c0 + kAttnChunk < p1) load_keys(c0 + kAttnChunk);
#pragma unroll
        for (int t = 0; t < kVB; ++t) {
          const int r = 16 * (t0 + t) + 4 * wave + rq;    // row within the chunk
          float vf[8];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            vf[2 * u] = __builtin_bit_cast(float, (uint32_t)vv[t][u] << 16);
            vf[2 * u + 1] = __builtin_bit_cast(float, (uint32_t)vv[t][u] & 0xffff0000u);
          }
#pragma unroll
          for (int g = 0; g < GM; ++g)
            if (g < G) {
              const float e = sc[g][r];
#pragma unroll
              for (int j = 0; j < 8; ++j) o[g][j] += e * vf[j];
            }
        }
      }
      __syncthreads();
    }
    // the four row groups of a wave (lanes 16 apart), then the four waves'
    // partial sums, then the softmax denominator
#pragma unroll
    for (int g = 0; g < GM; ++g)
      if (g < G) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          float v = o[g][j];
          v += __shfl_xor(v, 16);
          v += __shfl_xor(v, 32);
          if (rq == 0) part[wave][g][8 * cc + j] = v;
        }
      }
    __syncthreads();
    const size_t ps = (size_t)i * a.NS + split;          // this split's partial
    for (int x = tid; x < G * kHeadDim; x += kThreads) {
      const int g = x / kHeadDim, d = x % kHeadDim;
      st_coh(&a.po[ps * G * kHeadDim + x], ((part[0][g][d] + part[1][g][d]) + part[2][g][d]) + part[3][g][d]);
    }
    if (tid < G) {
      st_coh(&a.pml[(ps * G + tid) * 2], m_run[tid]);
      st_coh(&a.pml[(ps * G + tid) * 2 + 1], l_run[tid]);
    }
    if (sched == ET_SCHED_PER_OP) return true;
    wg_release();
    if (sched == ET_SCHED_BARRIER) {
      t0_notify_bcast(c, EV_ATT, EV_ATT, 1, N * a.NS, task);
    } else if (sched == ET_SCHED_STATIC) {
      t0_notify(c, a.ev_att + i, 1, a.NS, task);
    } else if (wg_notify(c, a.ev_att + i, 1, a.NS, task)) {
      wg_push(c, 1, [&](int) { return 2 * N + N * a.NS + i; }, [&](int) { return i; });
    }
    return true;
  };

  // merge of the NS splits of (b, h): the splits' running maxima rescale
  // their sums and outputs to the largest one (splits past the sequence's
  // length hold max -inf and contribute nothing)
  auto merge = [&](int i, int task) ET_INLINE -> bool {
    if (sched == ET_SCHED_STATIC) {
      if (!wg_wait(c, a.ev_att + i, a.NS, task)) return false;
    } else if (sched == ET_SCHED_BARRIER) {
      if (!wg_wait_bcast(c, EV_ATT, EV_ATT, task)) return false;
    }
    const int b = i / a.Hk, h = i % a.Hk;
    const size_t q0 = ((size_t)b * a.Hq + h * G) * kHeadDim;
    if (tid < G) {
      float M = -__builtin_inff();
      for (int j = 0; j < a.NS; ++j) M = fmaxf(M, ld_coh(&a.pml[(((size_t)i * a.NS + j) * G + tid) * 2]));
      float l = 0.f;
      for (int j = 0; j < a.NS; ++j) {
        const size_t q = ((size_t)i * a.NS + j) * G + tid;
        const float mj = ld_coh(&a.pml[q * 2]);
        const float w = mj == -__builtin_inff() ? 0.f : __expf(mj - M);
        l += w * ld_coh(&a.pml[q * 2 + 1]);
        sc[tid][j] = w;
      }
      l_run[tid] = l;
    }
    __syncthreads();
    for (int x = tid; x < G * kHeadDim; x += kThreads) {
      const int g = x / kHeadDim;
      float v = 0.f;
      for (int j = 0; j < a.NS; ++j)
        v += sc[g][j] * ld_coh(&a.po[((size_t)i * a.NS + j) * G * kHeadDim + x]);
      a.out[q0 + x] = v / l_run[g];
    }
    __syncthreads();
    return true;
  };

  // task -> (kind, i): static / dynamic interleave the branches (2i query,
  // 2i + 1 key); the baselines run all query tasks, then all key tasks
  auto run = [&](int t) ET_INLINE -> bool {
    if (t >= 2 * N + N * a.NS) return merge(t - 2 * N - N * a.NS, t);
    if (t >= 2 * N) return attention((t - 2 * N) / a.NS, (t - 2 * N) % a.NS, t);
    const int i = interleaved ? t >> 1 : t % N;
    const bool key = interleaved ? (t & 1) != 0 : t >= N;
    return key ? key_branch(i, t) : query_branch(i, t);
  };

  const int total = 2 * N + N * a.NS + N;
  if (sched == ET_SCHED_DYNAMIC) {
    bool ok = true;
    for (int t = c.wg; ok && t < ra.init_base; t += c.G) {
      const long long t0 = trace_now(c);
      ok = run(t);
      if (ok) count_run(c, t);
      if (ok) trace_task(c, t, t0);
    }
    PopState ps;
    while (ok) {
      const int t = wg_pop(c, ps);
      const long long t0 = trace_now(c);
      if (t < 0 || !run(t)) break;
      count_run(c, t);
      trace_task(c, t, t0);
    }
  } else if (sched == ET_SCHED_PER_OP) {
    // phases: query branch, key branch, attention splits, merges
    const int bounds[5] = {0, N, 2 * N, 2 * N + N * a.NS, 2 * N + N * a.NS + N};
    const int lo = bounds[ra.phase], hi = bounds[ra.phase + 1];
    for (int t = lo + c.wg; t < hi; t += c.G) {
      const long long t0 = trace_now(c);
      if (!run(t)) break;
      count_run(c, t);
      trace_task(c, t, t0);
    }
  } else {
    bool ok = true;
    for (int t = c.wg; ok && t < total; t += c.G) {
      const long long t0 = trace_now(c);
      ok = run(t);
      if (ok) count_run(c, t);
      if (ok) trace_task(c, t, t0);
    }
  }
  epilogue(c, total);
}

int launch_decode(const LaunchCommon& lc, const uint16_t* q, const uint16_t* k,
                  const uint16_t* v, const uint16_t* wq, const uint16_t* wk, const int* pos,
                  int B, float theta, float eps, uint16_t* kc, uint16_t* vc, int S, float* out) {
  const et_plan* p = lc.plan;
  DecodeArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.wq = wq;
  a.wk = wk;
  a.pos = pos;
  a.kc = kc;
  a.vc = vc;
  a.qr = reinterpret_cast<float*>(lc.ws + p->off_aux);
  // splits: enough ranges of the cache (a multiple of 64 positions each, at
  // most kMaxSplits) that the (sequence, head) pairs times the splits give
  // every workgroup a task; with as many pairs as workgroups, one split
  const int pairs = B * p->n_kv_heads;
  const int want = min(kMaxSplits, max(1, lc.G / pairs));
  const int L = cdiv(cdiv(S, want), 64) * 64;
  a.NS = cdiv(S, L);
  a.L = L;
  const size_t qr_floats = (size_t)p->max_tokens * p->n_heads * kHeadDim;
  a.po = a.qr + qr_floats;
  a.pml = a.po + kMaxSplits * qr_floats;
  a.out = out;
  a.B = B;
  a.Hq = p->n_heads;
  a.Hk = p->n_kv_heads;
  a.S = S;
  a.G = a.Hq / a.Hk;
  a.theta_log2 = (float)__builtin_log2((double)theta);
  a.eps = eps;
  const int N = B * a.Hk;
  a.ev_qk = EV_DEC_FIXED;
  a.ev_att = EV_DEC_FIXED + N;
  RunArgs ra = lc.run_args();
  ra.init_base = 2 * N < lc.G ? 2 * N : lc.G;   // dynamic: the first round of branch tasks runs directly
  ra.n_init = 2 * N - ra.init_base;              // the rest are implicit queue entries
  ra.total_hint = 2 * N + N * a.NS + N - ra.init_base;   // queue tasks: those and the pushed ones
  ra.extent = EV_DEC_FIXED + 2 * N;
  const void* kern = a.G <= 8 ? reinterpret_cast<const void*>(&decode_kernel<8>)
                              : reinterpret_cast<const void*>(&decode_kernel<16>);
  if (lc.sched == ET_SCHED_PER_OP) {
    for (int ph = 0; ph < 4; ++ph) {
      ra.phase = ph;
      const int e = lc.launch(kern, &ra, &a, false);
      if (e) return e;
    }
    return ET_OK;
  }
  return lc.launch(kern, &ra, &a, true);
}

}  // namespace et
