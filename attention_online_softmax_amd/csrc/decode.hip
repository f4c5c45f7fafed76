// Split-KV decode: one query token per (batch, query head) against a long
// contiguous KV cache.  The keys are cut into contiguous chunks; each chunk's
// unnormalised online-softmax state (m, l, acc) is computed independently and
// the states are folded with the monoid merge ("Tang, a compiler that derives
// GPU kernels and bounds how fast they can run", Abstract: online softmax as
// a monoid; "Compilers and Kernels", FlashAttention section, the recurrence's
// state and O_i = o_T / l_T).  Scoring one token is a matrix-vector product,
// so the split kernel is bound by streaming K and V from HBM: it reads each
// key/value row once for all query heads that share it.
#include "common.h"
#include "launch.h"

namespace attn {

template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static constexpr int PER16 = 4;  // elements per 16-byte access
  __device__ static void unpack(u32x4 x, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(x[i]);
  }
  __device__ static void store(float* p, const float* f) {
    *(f32x4*)p = f32x4{f[0], f[1], f[2], f[3]};
  }
};
template <>
struct Elem<uint16_t> {
  static constexpr int PER16 = 8;
  __device__ static void unpack(u32x4 x, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(x[i] << 16);
      f[2 * i + 1] = __uint_as_float(x[i] & 0xffff0000u);
    }
  }
  __device__ static void store(uint16_t* p, const float* f) {
    *(u32x4*)p = u32x4{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                       pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7])};
  }
};

constexpr int kDecodeThreads = 256;

// Grid: (n_splits, Hkv * n_hchunks, B).  Each workgroup owns one key chunk of
// one key/value head and up to GC of its query heads.
//   LPR lanes read one key row (16 bytes each), KPP rows are read per pass.
template <typename T, int D, int GC>
__global__ __launch_bounds__(kDecodeThreads) void decode_split_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    float* __restrict__ ws, int B, int Hq, int Hkv, int Skv, int chunk, int n_splits,
    int n_hchunks, float scale_log2) {
  constexpr int E = Elem<T>::PER16;
  constexpr int LPR = D / E;
  constexpr int KPP = kDecodeThreads / LPR;
  constexpr int MAXCHUNK = 1024;  // keys per workgroup held in LDS (host-checked)
  __shared__ float sP[GC][MAXCHUNK];
  __shared__ float sRed[KPP][D];
  __shared__ float sStat[GC][2];

  const int tid = threadIdx.x;
  const int split = blockIdx.x;
  const int hk = blockIdx.y / n_hchunks;
  const int hc = blockIdx.y % n_hchunks;
  const int b = blockIdx.z;
  const int G = Hq / Hkv;
  const int h0 = hk * G + hc * GC;         // first query head of this workgroup
  const int nh = min(GC, G - hc * GC);     // query heads handled here
  const int k_begin = min(split * chunk, Skv);
  const int k_end = min(k_begin + chunk, Skv);
  const int L = k_end - k_begin;
  const int64_t BHq = (int64_t)B * Hq;

  float* ws_m = ws;
  float* ws_l = ws + (int64_t)n_splits * BHq;
  float* ws_acc = ws + 2 * (int64_t)n_splits * BHq;

  if (L <= 0) {  // empty chunk: the identity state
    for (int i = tid; i < nh * D; i += kDecodeThreads) {
      const int hh = i / D, dd = i % D;
      const int64_t idx = (int64_t)split * BHq + (int64_t)b * Hq + h0 + hh;
      ws_acc[idx * D + dd] = 0.f;
      if (dd == 0) {
        ws_m[idx] = kNegInf;
        ws_l[idx] = 0.f;
      }
    }
    return;
  }

  const int sub = tid % LPR;   // which 16-byte column slice
  const int kr = tid / LPR;    // which key row of a pass
  const T* Kh = K + ((int64_t)(b * Hkv + hk) * Skv + k_begin) * D + sub * E;
  const T* Vh = V + ((int64_t)(b * Hkv + hk) * Skv + k_begin) * D + sub * E;

  // This lane's slice of each query head, pre-scaled into the log2 domain.
  float q[GC][E];
#pragma unroll
  for (int hh = 0; hh < GC; ++hh) {
    if (hh < nh) {
      const T* qp = Q + ((int64_t)b * Hq + h0 + hh) * D + sub * E;
      float f[E];
      Elem<T>::unpack(*(const u32x4*)qp, f);
#pragma unroll
      for (int e = 0; e < E; ++e) q[hh][e] = f[e] * scale_log2;
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) q[hh][e] = 0.f;
    }
  }

  // Phase 1: scores of every key in the chunk for every query head.
  constexpr int U = 4;  // passes in flight
  for (int p0 = 0; p0 < L; p0 += KPP * U) {
    u32x4 kx[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = p0 + u * KPP + kr;
      kx[u] = (r < L) ? *(const u32x4*)(Kh + (int64_t)r * D) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float f[E];
      Elem<T>::unpack(kx[u], f);
      const int r = p0 + u * KPP + kr;
#pragma unroll
      for (int hh = 0; hh < GC; ++hh) {
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) acc = fmaf(q[hh][e], f[e], acc);
#pragma unroll
        for (int w = 1; w < LPR; w <<= 1) acc += __shfl_xor(acc, w);
        if (sub == 0 && r < L && hh < nh) sP[hh][r] = acc;
      }
    }
  }
  __syncthreads();

  // Phase 2: per query head, chunk maximum m, p = exp2(s - m), l = sum p.
  const int lane = tid & 63, wave = tid >> 6;
  for (int hh = wave; hh < nh; hh += kDecodeThreads / 64) {
    float mx = kNegInf;
    for (int r = lane; r < L; r += 64) mx = fmaxf(mx, sP[hh][r]);
#pragma unroll
    for (int w = 32; w >= 1; w >>= 1) mx = fmaxf(mx, __shfl_xor(mx, w));
    float sum = 0.f;
    for (int r = lane; r < L; r += 64) {
      const float p = fast_exp2(sP[hh][r] - mx);
      sP[hh][r] = p;
      sum += p;
    }
#pragma unroll
    for (int w = 32; w >= 1; w >>= 1) sum += __shfl_xor(sum, w);
    if (lane == 0) {
      sStat[hh][0] = mx;
      sStat[hh][1] = sum;
    }
  }
  __syncthreads();

  // Phase 3: acc[h][:] = sum_r p[h][r] V[r][:], this lane's column slice and
  // every KPP-th key, then reduced over the KPP key groups through LDS.
  float acc[GC][E];
#pragma unroll
  for (int hh = 0; hh < GC; ++hh)
#pragma unroll
    for (int e = 0; e < E; ++e) acc[hh][e] = 0.f;
  for (int p0 = 0; p0 < L; p0 += KPP * U) {
    u32x4 vx[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = p0 + u * KPP + kr;
      vx[u] = (r < L) ? *(const u32x4*)(Vh + (int64_t)r * D) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = p0 + u * KPP + kr;
      if (r < L) {
        float f[E];
        Elem<T>::unpack(vx[u], f);
#pragma unroll
        for (int hh = 0; hh < GC; ++hh) {
          const float p = (hh < nh) ? sP[hh][r] : 0.f;
#pragma unroll
          for (int e = 0; e < E; ++e) acc[hh][e] = fmaf(p, f[e], acc[hh][e]);
        }
      }
    }
  }
  for (int hh = 0; hh < nh; ++hh) {
#pragma unroll
    for (int e = 0; e < E; ++e) sRed[kr][sub * E + e] = acc[hh][e];
    __syncthreads();
    const int64_t idx = (int64_t)split * BHq + (int64_t)b * Hq + h0 + hh;
    for (int dd = tid; dd < D; dd += kDecodeThreads) {
      float s = 0.f;
#pragma unroll 8
      for (int r = 0; r < KPP; ++r) s += sRed[r][dd];
      ws_acc[idx * D + dd] = s;
    }
    if (tid == 0) {
      ws_m[idx] = sStat[hh][0];
      ws_l[idx] = sStat[hh][1];
    }
    __syncthreads();
  }
}

// Grid: B * Hq workgroups of D threads.  Folds the n_splits states of one
// query with the monoid merge: every state is rescaled by exp2(m_s - M),
// M = max_s m_s (identity states, m_s = -inf, get weight 0), then O = acc / l
// and LSE = (M + log2 l) ln 2.
template <typename T, int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(const float* __restrict__ ws,
                                                           T* __restrict__ O,
                                                           float* __restrict__ LSE, int BHq,
                                                           int n_splits) {
  const int bh = blockIdx.x;
  const int dd = threadIdx.x;
  const float* ws_m = ws;
  const float* ws_l = ws + (int64_t)n_splits * BHq;
  const float* ws_acc = ws + 2 * (int64_t)n_splits * BHq;
  float M = kNegInf;
  for (int s = 0; s < n_splits; ++s) M = fmaxf(M, ws_m[(int64_t)s * BHq + bh]);
  float l = 0.f, a = 0.f;
  for (int s = 0; s < n_splits; ++s) {
    const float ms = ws_m[(int64_t)s * BHq + bh];
    const float w = (ms == kNegInf) ? 0.f : fast_exp2(ms - M);
    l = fmaf(w, ws_l[(int64_t)s * BHq + bh], l);
    a = fmaf(w, ws_acc[((int64_t)s * BHq + bh) * D + dd], a);
  }
  const float r = a / l;
  if constexpr (sizeof(T) == 4) {
    O[(int64_t)bh * D + dd] = r;
  } else {
    O[(int64_t)bh * D + dd] = f32_to_bf16(r);
  }
  if (LSE && dd == 0) LSE[bh] = (M + fast_log2(l)) * kLn2;
}

template <typename T, int D, int GC>
static hipError_t launch_decode_t(const DecodeArgs& a) {
  const int G = a.Hq / a.Hkv;
  const int n_hchunks = (G + GC - 1) / GC;
  const int chunk = (a.Skv + a.n_splits - 1) / a.n_splits;
  dim3 grid(a.n_splits, a.Hkv * n_hchunks, a.B);
  timing_mark(a.stream, 0);
  hipLaunchKernelGGL((decode_split_kernel<T, D, GC>), grid, dim3(kDecodeThreads), 0, a.stream,
                     (const T*)a.q, (const T*)a.k, (const T*)a.v, a.ws, a.B, a.Hq, a.Hkv, a.Skv,
                     chunk, a.n_splits, n_hchunks, a.scale * kLog2e);
  timing_mark(a.stream, 1);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  timing_mark(a.stream, 2);
  hipLaunchKernelGGL((decode_combine_kernel<T, D>), dim3(a.B * a.Hq), dim3(D), 0, a.stream,
                     (const float*)a.ws, (T*)a.o, a.lse, a.B * a.Hq, a.n_splits);
  timing_mark(a.stream, 3);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t dispatch_decode_g(const DecodeArgs& a) {
  const int G = a.Hq / a.Hkv;
  if (G == 1) return launch_decode_t<T, D, 1>(a);
  if (G == 2) return launch_decode_t<T, D, 2>(a);
  if (G <= 4) return launch_decode_t<T, D, 4>(a);
  return launch_decode_t<T, D, 8>(a);
}

template <typename T>
static hipError_t dispatch_decode_d(const DecodeArgs& a) {
  switch (a.d) {
    case 64: return dispatch_decode_g<T, 64>(a);
    case 128: return dispatch_decode_g<T, 128>(a);
    case 256: return dispatch_decode_g<T, 256>(a);
  }
  return hipErrorInvalidValue;
}

// Largest key chunk one split workgroup can hold (its LDS score buffer).
int decode_max_chunk() { return 1024; }

hipError_t launch_decode(const DecodeArgs& a) {
  return a.dtype == 0 ? dispatch_decode_d<float>(a) : dispatch_decode_d<uint16_t>(a);
}

}  // namespace attn
