// Projection GEMMs and their epilogues for the query side, the output side
// and the compression of the new token.
//
// Every projection on the decode path is a skinny product: a few rows of
// activations (one per sequence) against a large weight that is read once,
// so the kernels stream the weight at HBM rate and accumulate in fp32.
//   P[split][g][m][n] = sum over the split's k range of A_g[m][k] * W_g(n, k)
// with W_g(n, k) = W[g*sWg + n*ldw + k] ([out][in] weights, "NT") or
// W[g*sWg + k*ldw + n] (the transposed use of W_UK in the absorbed query,
// "NN"). Splitting k keeps the whole chip busy when the output is small; the
// epilogues sum the splits in a fixed order (deterministic) and apply what
// the step needs next (store, rotary embedding, latent norm + cache append).
//
// bf16 path: 256 threads, a 128 (n) x 32*MT (m) output tile, 64-deep k
// steps staged through LDS (register double buffering), bf16 MFMA 32x32x16
// with fp32 accumulation. fp32 path (and shapes the MFMA path does not take):
// one thread per output element.
#include "mla_internal.hpp"

namespace mla {
namespace {

constexpr int GBN = 128;   // n per workgroup
constexpr int GBK = 64;    // k per step
constexpr int GTH = 256;

// LDS slot (16-byte units) of chunk kc (8 k values) of tile row r; the XOR
// keeps 16 consecutive rows of one chunk on distinct bank groups.
__device__ __forceinline__ int gslot(int r, int kc) { return r * 8 + (kc ^ ((r >> 1) & 7)); }

struct GemmP {
  const void* A; long long lda, sAg;
  const uint16_t* W; long long ldw, sWg;
  int M, N, K, ksplit;    // ksplit = k per split (multiple of GBK)
  float* P;
};

template <int MT, bool A_F32, bool W_KN>
__global__ __launch_bounds__(GTH) void gemm_mfma_kernel(GemmP p) {
  __shared__ __align__(16) u32x4 wt[2][GBN * 8];
  __shared__ __align__(16) u32x4 at[2][32 * MT * 8];
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, h = lane >> 5, l32 = lane & 31;
  const int n0 = blockIdx.x * GBN;
  const int g = blockIdx.y;
  const int mblocks = (p.M + 32 * MT - 1) / (32 * MT);
  const int split = blockIdx.z / mblocks;
  const int m0 = (blockIdx.z % mblocks) * 32 * MT;
  const int k_begin = split * p.ksplit;
  const int k_end = min(p.K, k_begin + p.ksplit);
  const uint16_t* W = p.W + g * p.sWg;

  u32x4 wreg[4];
  u32x4 areg[MT];

  auto load_w = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (tid >> 3) + 32 * i, kc = tid & 7;
      const int n = n0 + r, k = k0 + 8 * kc;
      wreg[i] = (n < p.N && k < k_end)
                    ? *reinterpret_cast<const u32x4*>(W + static_cast<long long>(n) * p.ldw + k)
                    : u32x4{0u, 0u, 0u, 0u};
    }
  };
  // NN weights need an 8x8 transpose; keep their staging separate for clarity.
  u32x4 wkn[8];
  auto load_w_kn = [&](int k0) {
    const int kc = tid >> 4, nc = tid & 15;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int k = k0 + 8 * kc + i, n = n0 + 8 * nc;
      wkn[i] = (tid < 128 && k < k_end && n < p.N)
                   ? *reinterpret_cast<const u32x4*>(W + static_cast<long long>(k) * p.ldw + n)
                   : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto load_a = [&](int k0) {
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int r = (tid >> 3) + 32 * i, kc = tid & 7;
      const int m = m0 + r, k = k0 + 8 * kc;
      if (m < p.M && k < k_end) {
        if constexpr (A_F32) {
          const float* A = static_cast<const float*>(p.A) + g * p.sAg + static_cast<long long>(m) * p.lda + k;
          const f32x4 x0 = *reinterpret_cast<const f32x4*>(A);
          const f32x4 x1 = *reinterpret_cast<const f32x4*>(A + 4);
          areg[i] = u32x4{pack_bf16x2(x0[0], x0[1]), pack_bf16x2(x0[2], x0[3]),
                          pack_bf16x2(x1[0], x1[1]), pack_bf16x2(x1[2], x1[3])};
        } else {
          const uint16_t* A = static_cast<const uint16_t*>(p.A) + g * p.sAg + static_cast<long long>(m) * p.lda + k;
          areg[i] = *reinterpret_cast<const u32x4*>(A);
        }
      } else {
        areg[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto store_tiles = [&](int buf) {
    if constexpr (!W_KN) {
#pragma unroll
      for (int i = 0; i < 4; ++i) wt[buf][gslot((tid >> 3) + 32 * i, tid & 7)] = wreg[i];
    } else {
      if (tid < 128) {
        const int kc = tid >> 4, nc = tid & 15;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const unsigned sel = (j & 1) ? 0x07060302u : 0x05040100u;
          u32x4 o;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            o[q] = __builtin_amdgcn_perm(wkn[2 * q + 1][j >> 1], wkn[2 * q][j >> 1], sel);
          wt[buf][gslot(8 * nc + j, kc)] = o;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < MT; ++i) at[buf][gslot((tid >> 3) + 32 * i, tid & 7)] = areg[i];
  };

  f32x16 acc[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) acc[i] = f32x16{};

  if (k_begin < k_end) {
    if constexpr (W_KN) load_w_kn(k_begin); else load_w(k_begin);
    load_a(k_begin);
    store_tiles(0);
    __syncthreads();
    int buf = 0;
    for (int k0 = k_begin; k0 < k_end; k0 += GBK) {
      const bool more = k0 + GBK < k_end;
      if (more) {
        if constexpr (W_KN) load_w_kn(k0 + GBK); else load_w(k0 + GBK);
        load_a(k0 + GBK);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x4 av = wt[buf][gslot(32 * w + l32, 2 * j + h)];
#pragma unroll
        for (int i = 0; i < MT; ++i) {
          const u32x4 bv = at[buf][gslot(32 * i + l32, 2 * j + h)];
          acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av),
                                                           __builtin_bit_cast(bf16x8, bv), acc[i],
                                                           0, 0, 0);
        }
      }
      if (more) store_tiles(buf ^ 1);
      __syncthreads();
      buf ^= 1;
    }
  }
  // D[n][m]: lane holds m = 32i + l32, n = 32w + 8(r/4) + 4h + r%4.
  float* P = p.P + (static_cast<long long>(split) * gridDim.y + g) * p.M * p.N;
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int m = m0 + 32 * i + l32;
    if (m >= p.M) continue;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int n = n0 + 32 * w + 8 * q + 4 * h;
      float* dst = P + static_cast<long long>(m) * p.N + n;
      if (n + 3 < p.N) {
        *reinterpret_cast<f32x4*>(dst) =
            f32x4{acc[i][4 * q], acc[i][4 * q + 1], acc[i][4 * q + 2], acc[i][4 * q + 3]};
      } else {
        for (int e = 0; e < 4 && n + e < p.N; ++e) dst[e] = acc[i][4 * q + e];
      }
    }
  }
}

// One thread per output element (fp32 storage, or shapes the MFMA kernel
// does not take). Same partial layout as the MFMA kernel.
template <typename TA, typename TW>
__global__ __launch_bounds__(256) void gemm_simt_kernel(const TA* __restrict__ A, long long lda,
                                                         long long sAg, const TW* __restrict__ W,
                                                         long long ldw, long long sWg, int w_kn,
                                                         int M, int N, int K, int G, int ksplit,
                                                         float* __restrict__ P) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  const int m = blockIdx.y;
  const int g = blockIdx.z % G;
  const int split = blockIdx.z / G;
  if (n >= N) return;
  const int k0 = split * ksplit, k1 = min(K, k0 + ksplit);
  const TA* a = A + g * sAg + static_cast<long long>(m) * lda;
  const TW* wp = W + g * sWg;
  float acc = 0.f;
  if (!w_kn) {
    const TW* wr = wp + static_cast<long long>(n) * ldw;
    for (int k = k0; k < k1; ++k) acc += Elem<TA>::ld(a + k) * Elem<TW>::ld(wr + k);
  } else {
    for (int k = k0; k < k1; ++k) acc += Elem<TA>::ld(a + k) * Elem<TW>::ld(wp + static_cast<long long>(k) * ldw + n);
  }
  P[((static_cast<long long>(split) * G + g) * M + m) * N + n] = acc;
}

template <typename TO>
__global__ void reduce_store_kernel(const float* __restrict__ P, int splits, int G, int M, int N,
                                    TO* __restrict__ out, long long ldo, long long sOg) {
  const long long idx = blockIdx.x * 256LL + threadIdx.x;
  const long long total = static_cast<long long>(G) * M * N;
  if (idx >= total) return;
  const int n = static_cast<int>(idx % N);
  const int m = static_cast<int>((idx / N) % M);
  const int g = static_cast<int>(idx / (static_cast<long long>(N) * M));
  float v = 0.f;
  for (int s = 0; s < splits; ++s) v += P[s * total + idx];
  Elem<TO>::st(out + g * sOg + m * ldo + n, v);
}

// Rotary projection [M][G*d_R] -> rotated, stored at out[m*ldo + g*sOg + j].
template <typename TO>
__global__ void reduce_rope_kernel(const float* __restrict__ P, int splits, int M, int G, int d_R,
                                   const int32_t* __restrict__ pos, float theta,
                                   TO* __restrict__ out, long long ldo, long long sOg) {
  const long long idx = blockIdx.x * 256LL + threadIdx.x;   // pair index
  const int half = d_R / 2;
  const long long total_pairs = static_cast<long long>(M) * G * half;
  if (idx >= total_pairs) return;
  const int j = static_cast<int>(idx % half);
  const int g = static_cast<int>((idx / half) % G);
  const int m = static_cast<int>(idx / (static_cast<long long>(half) * G));
  const long long total = static_cast<long long>(M) * G * d_R;
  const long long e0 = (static_cast<long long>(m) * G + g) * d_R + 2 * j;
  float x0 = 0.f, x1 = 0.f;
  for (int s = 0; s < splits; ++s) {
    x0 += P[s * total + e0];
    x1 += P[s * total + e0 + 1];
  }
  float c, sn;
  rope_cs(pos[m], j, d_R, theta, &c, &sn);
  TO* o = out + m * ldo + g * sOg + 2 * j;
  Elem<TO>::st(o, x0 * c - x1 * sn);
  Elem<TO>::st(o + 1, x0 * sn + x1 * c);
}

// One workgroup per sequence: sum the splits of [c ; k_R], optionally
// RMS-normalise c ("Understanding MLA" (Dong), A2: norm on the latent only),
// rotate k_R at the token's position, round and write the cache row.
template <typename T>
__global__ __launch_bounds__(256) void append_kernel(const float* __restrict__ Pc, int splits_c,
                                                     const float* __restrict__ Pr, int splits_r, int M,
                                                     int d_c, int d_R, const T* __restrict__ gamma,
                                                     float eps, const int32_t* __restrict__ pos,
                                                     float theta, mla_cache cache) {
  extern __shared__ float row[];    // d_c + d_R floats, then 4 for the reduction
  const int m = blockIdx.x;
  const int D = d_c + d_R;
  float* red = row + D;
  float ss = 0.f;
  for (int c = threadIdx.x; c < d_c; c += blockDim.x) {
    float v = 0.f;
    for (int s = 0; s < splits_c; ++s) v += Pc[(static_cast<long long>(s) * M + m) * d_c + c];
    row[c] = v;
    ss += v * v;
  }
  for (int c = threadIdx.x; c < d_R; c += blockDim.x) {
    float v = 0.f;
    for (int s = 0; s < splits_r; ++s) v += Pr[(static_cast<long long>(s) * M + m) * d_R + c];
    row[d_c + c] = v;
  }
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) tot += red[i];
  const float rinv = gamma ? rsqrtf(tot / d_c + eps) : 1.f;
  const int t = pos[m];
  T* dst;
  if (cache.block_table == nullptr) {
    dst = static_cast<T*>(cache.data) + (static_cast<long long>(m) * cache.capacity + t) * D;
  } else {
    const int blk = cache.block_table[m * cache.max_blocks + t / cache.block_size];
    dst = static_cast<T*>(cache.data) +
          (static_cast<long long>(blk) * cache.block_size + t % cache.block_size) * D;
  }
  for (int c = threadIdx.x; c < d_c; c += blockDim.x) {
    float v = row[c];
    if (gamma) v = v * rinv * Elem<T>::ld(gamma + c);
    Elem<T>::st(dst + c, v);
  }
  for (int j = threadIdx.x; j < d_R / 2; j += blockDim.x) {
    float c, s;
    rope_cs(t, j, d_R, theta, &c, &s);
    const float x0 = row[d_c + 2 * j], x1 = row[d_c + 2 * j + 1];
    Elem<T>::st(dst + d_c + 2 * j, x0 * c - x1 * s);
    Elem<T>::st(dst + d_c + 2 * j + 1, x0 * s + x1 * c);
  }
}

bool mfma_ok(const GemmArgs& a) {
  if (a.dtype != MLA_BF16) return false;
  if (a.K % 8 || a.lda % 8 || a.ldw % 8 || a.sAg % 8 || a.sWg % 8) return false;
  if (a.w_kn && a.N % 8) return false;
  if ((reinterpret_cast<uintptr_t>(a.A) | reinterpret_cast<uintptr_t>(a.W)) & 15) return false;
  return true;
}

int device_cus() {
  static thread_local int dev_cached = -1, cus = 256;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return cus;
  if (dev != dev_cached) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
    dev_cached = dev;
  }
  return cus;
}

}  // namespace

int gemm_splits(int M, int N, int K, int G, int dtype) {
  (void)dtype;
  const int ksteps = (K + GBK - 1) / GBK;
  const int mblocks = (M + 127) / 128;
  const long long tiles = static_cast<long long>((N + GBN - 1) / GBN) * G * mblocks;
  const long long target = 2LL * 256;   // about two workgroups per compute unit
  long long s = (target + tiles - 1) / tiles;
  if (s > ksteps) s = ksteps;
  if (s < 1) s = 1;
  // k per split is a whole number of steps; recompute the count that covers K
  const int kper = static_cast<int>((ksteps + s - 1) / s) * GBK;
  return (K + kper - 1) / kper;
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream) {
  const int splits = a.splits;
  const int ksteps = (a.K + GBK - 1) / GBK;
  const int kper = ((ksteps + splits - 1) / splits) * GBK;
  if (mfma_ok(a)) {
    GemmP p{a.A, a.lda, a.sAg, static_cast<const uint16_t*>(a.W), a.ldw, a.sWg, a.M, a.N, a.K, kper, a.P};
    const int MT = a.M <= 32 ? 1 : a.M <= 64 ? 2 : 4;
    const int mblocks = (a.M + 32 * MT - 1) / (32 * MT);
    const dim3 grid((a.N + GBN - 1) / GBN, a.G, splits * mblocks);
#define MLA_GEMM(MTV)                                                                            \
  if (a.a_f32) {                                                                                 \
    if (a.w_kn) gemm_mfma_kernel<MTV, true, true><<<grid, GTH, 0, stream>>>(p);                  \
    else gemm_mfma_kernel<MTV, true, false><<<grid, GTH, 0, stream>>>(p);                        \
  } else {                                                                                       \
    if (a.w_kn) gemm_mfma_kernel<MTV, false, true><<<grid, GTH, 0, stream>>>(p);                 \
    else gemm_mfma_kernel<MTV, false, false><<<grid, GTH, 0, stream>>>(p);                       \
  }
    if (MT == 1) { MLA_GEMM(1) } else if (MT == 2) { MLA_GEMM(2) } else { MLA_GEMM(4) }
#undef MLA_GEMM
    return hipGetLastError();
  }
  const dim3 grid((a.N + 255) / 256, a.M, a.G * splits);
  if (a.dtype == MLA_BF16) {
    const uint16_t* W = static_cast<const uint16_t*>(a.W);
    if (a.a_f32)
      gemm_simt_kernel<float, uint16_t><<<grid, 256, 0, stream>>>(
          static_cast<const float*>(a.A), a.lda, a.sAg, W, a.ldw, a.sWg, a.w_kn, a.M, a.N, a.K, a.G, kper, a.P);
    else
      gemm_simt_kernel<uint16_t, uint16_t><<<grid, 256, 0, stream>>>(
          static_cast<const uint16_t*>(a.A), a.lda, a.sAg, W, a.ldw, a.sWg, a.w_kn, a.M, a.N, a.K, a.G, kper, a.P);
  } else {
    gemm_simt_kernel<float, float><<<grid, 256, 0, stream>>>(
        static_cast<const float*>(a.A), a.lda, a.sAg, static_cast<const float*>(a.W), a.ldw, a.sWg,
        a.w_kn, a.M, a.N, a.K, a.G, kper, a.P);
  }
  return hipGetLastError();
}

hipError_t launch_reduce_store(const float* P, int splits, int G, int M, int N, void* out,
                               long long ldo, long long sOg, int out_dtype, hipStream_t stream) {
  const long long total = static_cast<long long>(G) * M * N;
  const dim3 grid(static_cast<unsigned>((total + 255) / 256));
  if (out_dtype == MLA_BF16)
    reduce_store_kernel<uint16_t><<<grid, 256, 0, stream>>>(P, splits, G, M, N, static_cast<uint16_t*>(out), ldo, sOg);
  else
    reduce_store_kernel<float><<<grid, 256, 0, stream>>>(P, splits, G, M, N, static_cast<float*>(out), ldo, sOg);
  return hipGetLastError();
}

hipError_t launch_reduce_rope(const float* P, int splits, int M, int G, int d_R, const int32_t* pos,
                              float theta, void* out, long long ldo, long long sOg, int out_dtype,
                              hipStream_t stream) {
  const long long pairs = static_cast<long long>(M) * G * (d_R / 2);
  const dim3 grid(static_cast<unsigned>((pairs + 255) / 256));
  if (out_dtype == MLA_BF16)
    reduce_rope_kernel<uint16_t><<<grid, 256, 0, stream>>>(P, splits, M, G, d_R, pos, theta, static_cast<uint16_t*>(out), ldo, sOg);
  else
    reduce_rope_kernel<float><<<grid, 256, 0, stream>>>(P, splits, M, G, d_R, pos, theta, static_cast<float*>(out), ldo, sOg);
  return hipGetLastError();
}

hipError_t launch_append(const float* Pc, int splits_c, const float* Pr, int splits_r, int M, int d_c, int d_R,
                         const void* gamma, float eps, const int32_t* pos, float theta,
                         const mla_cache& cache, int dtype, hipStream_t stream) {
  const size_t shmem = (static_cast<size_t>(d_c + d_R) + 8) * sizeof(float);
  if (dtype == MLA_BF16)
    append_kernel<uint16_t><<<M, 256, shmem, stream>>>(Pc, splits_c, Pr, splits_r, M, d_c, d_R,
                                                       static_cast<const uint16_t*>(gamma), eps, pos, theta, cache);
  else
    append_kernel<float><<<M, 256, shmem, stream>>>(Pc, splits_c, Pr, splits_r, M, d_c, d_R,
                                                    static_cast<const float*>(gamma), eps, pos, theta, cache);
  return hipGetLastError();
}


}  // namespace mla
