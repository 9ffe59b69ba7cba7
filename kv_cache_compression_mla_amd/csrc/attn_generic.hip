// General-geometry latent attention (any d_c, d_R, H; fp32 or bf16 storage)
// and the cross-split combine shared by both attention kernels.
//
// Same computation as the MFMA kernel: for each sequence b and head i,
// s(u) = scale * (q(b,i) . row(b,u)) over the full row, softmax over the rows
// attended, o_lat = sum_u p(u) row(b,u)[0:d_c] ("Understanding MLA" (Dong),
// section 4 regrouping; aicassindra MLA explainer, "End-to-end flow").
// One workgroup per (sequence, split, head), plain fp32 arithmetic. Partials
// use the same convention as the MFMA kernel: m in log2 units (score *
// scale * log2 e) and l = sum 2^(score' - m).
#include "mla_internal.hpp"

namespace mla {
namespace {

constexpr int GT = 256;          // threads per workgroup
constexpr int MAX_DC_PER_T = 4;  // d_c <= 1024

// Row of entry u of sequence b: position u, or the listed position
// indices[b][u] for sparse attention.
template <typename T>
__device__ __forceinline__ const T* g_row_ptr(const T* cache, const int32_t* table, long long cap,
                                              int bs, int maxb, int D, int b, int u, const int32_t* indices,
                                              int topk) {
  if (indices) u = indices[static_cast<long long>(b) * topk + u];
  if (table == nullptr) return cache + (b * cap + u) * static_cast<long long>(D);
  const int blk = table[b * maxb + u / bs];
  return cache + (static_cast<long long>(blk) * bs + u % bs) * D;
}

__device__ __forceinline__ float block_max(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < GT / 64; ++i) r = fmaxf(r, red[i]);
  __syncthreads();
  return r;
}

__device__ __forceinline__ float block_sum(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = 0.f;
  for (int i = 0; i < GT / 64; ++i) r += red[i];
  __syncthreads();
  return r;
}

template <typename T>
__global__ __launch_bounds__(GT) void attn_generic_kernel(AttnArgs a) {
  extern __shared__ float sh[];        // q[D] | p[GT] | red[4]
  const int D = a.d_c + a.d_R;
  float* qs = sh;
  float* ps = sh + D;
  float* red = ps + GT;
  const int head = blockIdx.x % a.H;
  const int s_idx = (blockIdx.x / a.H) % a.splits;
  const int b = blockIdx.x / (a.H * a.splits);
  const int tid = threadIdx.x;
  // query row [q_lat ; q_R ; low term of q_R]: the rotary part is the sum
  const T* q = static_cast<const T*>(a.q) + (static_cast<long long>(b) * a.H + head) * (D + a.d_R);
  const T* cache = static_cast<const T*>(a.cache);
  for (int k = tid; k < D; k += GT) qs[k] = Elem<T>::ld(q + k) + (k >= a.d_c ? Elem<T>::ld(q + k + a.d_R) : 0.f);
  const int L = virt_len(a.seq_lens, b, a.qpt);
  const int bc = a.qpt == 1 ? b : b / a.qpt;   // the cached sequence it reads
  const int r0 = s_idx * a.chunk;
  const int r1 = min(r0 + a.chunk, L);
  const float sl2 = a.scale * 1.4426950408889634f;
  __syncthreads();

  float m = -INFINITY, l = 0.f;
  float acc[MAX_DC_PER_T];
#pragma unroll
  for (int j = 0; j < MAX_DC_PER_T; ++j) acc[j] = 0.f;

  for (int base = r0; base < r1; base += GT) {
    const int u = base + tid;
    float sc = -INFINITY;
    if (u < r1) {
      const T* row = g_row_ptr(cache, a.block_table, a.capacity, a.block_size, a.max_blocks, D, bc, u, a.indices,
                               a.topk);
      float dot = 0.f;
      for (int k = 0; k < D; ++k) dot += qs[k] * Elem<T>::ld(row + k);
      sc = dot * sl2;
    }
    const float bm = block_max(sc, red);
    const float m_new = fmaxf(m, bm);
    const float alpha = exp2f(m - m_new);
    const float pv = (u < r1) ? exp2f(sc - m_new) : 0.f;
    ps[tid] = pv;
    const float bs = block_sum(pv, red);   // also orders the ps writes before the reads below
    l = l * alpha + bs;
    m = m_new;
    const int nrow = min(GT, r1 - base);
#pragma unroll
    for (int j = 0; j < MAX_DC_PER_T; ++j) {
      const int c = tid + j * GT;
      if (c < a.d_c) {
        float x = acc[j] * alpha;
        for (int t = 0; t < nrow; ++t) {
          const T* row = g_row_ptr(cache, a.block_table, a.capacity, a.block_size, a.max_blocks, D, bc,
                                   base + t, a.indices, a.topk);
          x += ps[t] * Elem<T>::ld(row + c);
        }
        acc[j] = x;
      }
    }
    __syncthreads();
  }

  if (a.splits == 1) {
    float* o = a.o_lat + (static_cast<long long>(b) * a.H + head) * a.d_c;
    const float inv = (l > 0.f) ? 1.f / l : 0.f;
#pragma unroll
    for (int j = 0; j < MAX_DC_PER_T; ++j) {
      const int c = tid + j * GT;
      if (c < a.d_c) o[c] = acc[j] * inv;
    }
    if (a.lse && tid == 0)
      a.lse[b * a.H + head] = (l > 0.f) ? (m + log2f(l)) * 0.69314718055994531f : -INFINITY;
  } else if (r0 < r1) {
    const long long pidx = (static_cast<long long>(b) * a.splits + s_idx) * a.H + head;
    float* o = a.part_o + pidx * a.d_c;
#pragma unroll
    for (int j = 0; j < MAX_DC_PER_T; ++j) {
      const int c = tid + j * GT;
      if (c < a.d_c) o[c] = acc[j];
    }
    if (tid == 0) {
      a.part_ml[pidx * 2] = m;
      a.part_ml[pidx * 2 + 1] = l;
    }
  }
}

// Exact merge of per-split softmax partials (m_s, l_s, O_s) of one (b, head):
// with M = max m_s and w_s = 2^(m_s - M),  o = sum w_s O_s / sum w_s l_s.
// Splits that start at or past the sequence length hold no partial.
__global__ __launch_bounds__(128) void attn_combine_kernel(AttnArgs a) {
  const int head = blockIdx.x % a.H;
  const int b = blockIdx.x / a.H;
  const int L = virt_len(a.seq_lens, b, a.qpt);
  const int nv = min(a.splits, (L + a.chunk - 1) / a.chunk);
  float* o = a.o_lat + (static_cast<long long>(b) * a.H + head) * a.d_c;
  const long long base = static_cast<long long>(b) * a.splits * a.H + head;   // split 0
  float M = -INFINITY;
  for (int s = 0; s < nv; ++s) M = fmaxf(M, a.part_ml[(base + static_cast<long long>(s) * a.H) * 2]);
  float den = 0.f;
  for (int s = 0; s < nv; ++s) {
    const long long pi = base + static_cast<long long>(s) * a.H;
    den += exp2f(a.part_ml[pi * 2] - M) * a.part_ml[pi * 2 + 1];
  }
  const float inv = (den > 0.f) ? 1.f / den : 0.f;
  if ((a.d_c & 3) == 0) {
    // four columns per thread, streamed once (partials are not reused)
    for (int c = 4 * threadIdx.x; c < a.d_c; c += 4 * blockDim.x) {
      f32x4 x = {0.f, 0.f, 0.f, 0.f};
      for (int s = 0; s < nv; ++s) {
        const long long pi = base + static_cast<long long>(s) * a.H;
        const float ws = exp2f(a.part_ml[pi * 2] - M);
        x += ws * __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(a.part_o + pi * a.d_c + c));
      }
      *reinterpret_cast<f32x4*>(o + c) = x * inv;
    }
  } else {
    for (int c = threadIdx.x; c < a.d_c; c += blockDim.x) {
      float x = 0.f;
      for (int s = 0; s < nv; ++s) {
        const long long pi = base + static_cast<long long>(s) * a.H;
        x += exp2f(a.part_ml[pi * 2] - M) * a.part_o[pi * a.d_c + c];
      }
      o[c] = x * inv;
    }
  }
  if (a.lse && threadIdx.x == 0)
    a.lse[b * a.H + head] = (den > 0.f) ? (M + log2f(den)) * 0.69314718055994531f : -INFINITY;
}

}  // namespace

hipError_t launch_attn_generic(const AttnArgs& a, hipStream_t stream) {
  const size_t shmem = (static_cast<size_t>(a.d_c + a.d_R) + GT + 8) * sizeof(float);
  const dim3 grid(a.B * a.splits * a.H);
  if (a.dtype == MLA_BF16)
    attn_generic_kernel<uint16_t><<<grid, GT, shmem, stream>>>(a);
  else
    attn_generic_kernel<float><<<grid, GT, shmem, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_attn_combine(const AttnArgs& a, hipStream_t stream) {
  attn_combine_kernel<<<dim3(a.B * a.H), 128, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace mla
