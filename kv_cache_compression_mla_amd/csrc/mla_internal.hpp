// Internal declarations shared by the HIP translation units of libmla.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla.h"

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Scalar conversions (bf16 is carried as uint16_t bit patterns in memory).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
// Round to nearest, ties to even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}
// Two floats -> packed bf16 pair (lo = a, hi = b), nearest-even: one
// v_cvt_pk_bf16_f32 on gfx950 (same rounding as f32_to_bf16 for every
// non-NaN value; NaN stays NaN).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef float v2f __attribute__((ext_vector_type(2)));
  typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f{a, b}), v2bf));
}

// An fp32 activation carried into a bf16 MFMA as two bf16 terms: hi = the
// nearest bf16 of x, lo = the nearest bf16 of x - hi (exact in fp32). hi + lo
// equals x to about 2^-17 relative, so a product summed over both terms
// keeps the activation's fp32 precision (the weights are bf16 already). Used
// for the intermediate activations of the query and output sides, whose
// rounding to bf16 would otherwise feed every head's scores.
__device__ __forceinline__ void split_bf16x2(float a, float b, uint32_t* hi, uint32_t* lo) {
  const uint32_t h = pack_bf16x2(a, b);
  *hi = h;
  *lo = pack_bf16x2(a - __uint_as_float(h << 16), b - __uint_as_float(h & 0xffff0000u));
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ static __forceinline__ float ld(const float* p) { return *p; }
  __device__ static __forceinline__ void st(float* p, float v) { *p = v; }
};
template <> struct Elem<uint16_t> {
  __device__ static __forceinline__ float ld(const uint16_t* p) { return bf16_to_f32(*p); }
  __device__ static __forceinline__ void st(uint16_t* p, float v) { *p = f32_to_bf16(v); }
};

// Rotary angle cos/sin for pair j of a d_R-wide vector at integer position
// pos: angle = pos * theta^(-2j/d_R). The angle (up to ~3e4 rad at long
// contexts) is formed and reduced to [-pi, pi] in double: the frequency as
// exp2(-(2j/d_R) log2 theta), then Cody-Waite reduction by a two-part 2*pi
// (a rounded multiple k of 2*pi removed with two fused multiply-adds), so the
// reduced angle is accurate to ~1e-12 rad; float32 sincos of it is then
// accurate to about one float32 ulp, far below the bf16 rounding of the
// rotated values.
__device__ __forceinline__ void rope_cs(int pos, int j, int d_R, float theta, float* c, float* s) {
  const double inv = exp2(-(2.0 * j / d_R) * log2(static_cast<double>(theta)));
  const double a = static_cast<double>(pos) * inv;
  constexpr double kTwoPiHi = 6.283185307179586;          // double nearest 2*pi
  constexpr double kTwoPiLo = 2.4492935982947064e-16;     // 2*pi - kTwoPiHi
  const double k = rint(a * (1.0 / kTwoPiHi));
  const double r = fma(-k, kTwoPiLo, fma(-k, kTwoPiHi, a));
  sincosf(static_cast<float>(r), s, c);
}

// ---------------------------------------------------------------------------
// Launchers implemented in the .hip files (all enqueue on `stream`).
// ---------------------------------------------------------------------------

// Partial-sum GEMM: P[split][g][m][n] = sum over the split's k range of
// A_g[m][k] * W_g(n, k); W_g(n, k) = W[g*sWg + n*ldw + k] (w_kn == false) or
// W[g*sWg + k*ldw + n] (w_kn == true). Element types by dtype.
struct GemmArgs {
  const void* A;  long long lda, sAg;  bool a_f32;   // A element: f32 or storage dtype
  const void* W;  long long ldw, sWg;  bool w_kn;
  int M, N, K, G;
  int splits;                 // k splits (>= 1)
  float* P;                   // [splits][G][M][N] fp32
  int dtype;                  // storage dtype of W (and of A unless a_f32)
  // Optional direct store (taken when gemm_direct() says so): the product is
  // written to out[g*sOg + m*ldo + n] in out_dtype instead of partials P.
  void* out = nullptr;
  long long ldo = 0, sOg = 0;
  int out_dtype = 0;
  // Optional second weight (G = 1, streaming kernel only): output columns
  // n >= n_split read W2 row n - n_split (same ldw), so two products of one
  // activation run as one launch.
  const void* W2 = nullptr;
  int n_split = 0;
  // float32 activations (a_f32) as two bf16 terms (split_bf16x2): about
  // float32 precision for twice the MFMAs; otherwise rounded once to bf16
  bool a_split = false;
};
hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream);
// True when launch_gemm stores a's product directly to a.out (one split on
// the streaming kernel); otherwise it writes partials for an epilogue.
bool gemm_direct(const GemmArgs& a);
// True when launch_gemm can take a's second weight (W2, n_split).
bool gemm_concat_ok(const GemmArgs& a);
// Tall bf16 products stored directly (out set; the P, splits and W2 fields
// are not used): more than 128 rows of A, NT weights, K a multiple of 64.
bool gemm_tall_ok(const GemmArgs& a);
hipError_t launch_gemm_tall(const GemmArgs& a, hipStream_t stream);
// Number of k splits launch_gemm would pick for a shape (used to size workspaces).
int gemm_splits(int M, int N, int K, int G, int dtype);

// Sum the splits of P and store to a strided output in dtype out_dtype:
// out[g*sOg + m*ldo + n] = sum_s P[s][g][m][n].
hipError_t launch_reduce_store(const float* P, int splits, int G, int M, int N,
                               void* out, long long ldo, long long sOg, int out_dtype,
                               hipStream_t stream);
// Sum splits of an [M][N] product (G = 1, rows N apart) into out32 (float32)
// and out16 (the same sums rounded to bf16).
hipError_t launch_reduce_store_dual(const float* P, int splits, int M, int N, float* out32, uint16_t* out16,
                                    hipStream_t stream);
// Sum splits of the rotary projection [M][G*d_R] (g = head), rotate each head's
// d_R vector at pos[m], store to out[m*ldo + g*sOg + j] as two terms of the
// storage type: the nearest value, and at j + d_R the nearest value of the
// remainder.
hipError_t launch_reduce_rope(const float* P, int splits, int M, int G, int d_R,
                              const int32_t* pos, float theta, void* out,
                              long long ldo, long long sOg, int out_dtype,
                              hipStream_t stream);
// Sum splits of the latent [M][d_c] and rotary key [M][d_R] partials,
// optionally RMS-normalise the latent, rotate the key at pos[m], round, and
// write the row to the cache at position pos[m].
hipError_t launch_append(const float* Pc, int splits_c, int ldc, const float* Pr, int splits_r, int ldr, int M,
                         int d_c, int d_R, const void* gamma, float eps, const int32_t* pos,
                         float theta, const mla_cache& cache, int dtype, hipStream_t stream);

// Copy n rotary query vectors (d_R values at src + k*lds + off_src) into the
// absorbed query rows at dst + k*ldd + off_dst, each followed by a zero
// second term.
hipError_t launch_rope_query_copy(const void* src, long long lds, int off_src, void* dst, long long ldd, int off_dst,
                                  int d_R, long long n, int dtype, hipStream_t stream);

// Offline composition C(g, m, n) = sum_k X(g, k, m) Y(g, k, n) with element
// strides (see gemm.hip); fp32 accumulation, stored in dtype.
hipError_t launch_compose(const void* X, long long xg, long long xk, long long xm, const void* Y, long long yg,
                          long long yk, void* C, long long cg, long long cm, int G, int M, int N, int K, int dtype,
                          hipStream_t stream);

// Attention. chunk = rows per split (multiple of 32 for the MFMA kernel).
struct AttnArgs {
  const void* q;
  const void* cache;
  const int32_t* block_table;
  long long capacity;
  int block_size, max_blocks;
  const int32_t* seq_lens;
  int B, H, d_c, d_R;
  int chunk, splits;
  float scale;
  float* o_lat;
  float* lse;
  float* part_o;    // generic: [B][splits][H][d_c] fp32; MFMA: [grid][H][d_c] fp16 (scaled), by chunk
  float* part_ml;   // generic: [B][splits][H][2];        MFMA: [grid][H][4] (m, l, E, unused)
  int dtype;
  // MFMA kernel: workgroups launched, and per sequence (first chunk, chunks)
  // of the plan it computes on the device (splits = 0: balanced plan)
  int grid = 0;
  int2* plan_seq = nullptr;
  // sparse attention: entry u of sequence b is the row at indices[b*topk + u]
  // (seq_lens then holds the entry counts)
  const int32_t* indices = nullptr;
  int topk = 0;
  // causal prefill in the absorbed form: B counts query tokens, qpt of them
  // per cached sequence; entry b attends the first virt_len(...) rows of
  // sequence b / qpt
  int qpt = 1;
  // kernel-timing events for one call (mla_time_next_attn), NULL for none:
  // t_start takes the attention kernel's start, t_kernel_end its end and
  // t_call_end the end of the call's last kernel
  hipEvent_t t_start = nullptr, t_kernel_end = nullptr, t_call_end = nullptr;
};

// Rows attended by entry b: seq_lens[b] for decode (qpt = 1); with qpt query
// tokens per sequence, token t = b % qpt of sequence b / qpt sits at position
// seq_lens - qpt + t and attends the rows up to and including it.
__device__ __forceinline__ int virt_len(const int32_t* seq_lens, int b, int qpt) {
  if (qpt == 1) return seq_lens[b];
  return max(0, seq_lens[b / qpt] - (qpt - 1 - b % qpt));
}
// Causal prefill attention in the materialised form: keys and values expanded
// per head from the cached latents, T query tokens per sequence, token t at
// position seq_lens[b] - T + t attending rows 0..that position.
struct PrefillArgs {
  const void* q;            // [B][T][H][d_h + d_R]: per head [q_C ; q_R]
  const void* K;            // [cache storage rows][H][d_h]: expanded keys (nope part)
  const void* Vt;           // [H][d_v][vt_ld]: expanded values, transposed
  long long vt_ld;          // row length of Vt
  long long vt_seq;         // contiguous cache: Vt column of row u of sequence b is b*vt_seq + u
  const void* cache;        // latent rows [c ; k_R]; the rotary keys are read here
  const int32_t* block_table;
  long long capacity;
  int block_size, max_blocks;
  const int32_t* seq_lens;  // rows per sequence, the T tokens' own rows included
  int B, T, H, d_h, d_v, d_c, d_R;
  float scale;
  void* o;                  // [B][T][H][d_v] storage dtype
  float* lse;               // [B][T][H] or NULL
  int dtype;
};
// MFMA kernel: bf16, d_h = d_v = 128, d_R = 64, contiguous or block_size >= 8.
hipError_t launch_prefill_mfma(const PrefillArgs& a, hipStream_t stream);
hipError_t launch_prefill_generic(const PrefillArgs& a, hipStream_t stream);

hipError_t launch_attn_mfma(const AttnArgs& a, hipStream_t stream);
hipError_t launch_attn_generic(const AttnArgs& a, hipStream_t stream);
hipError_t launch_attn_combine(const AttnArgs& a, hipStream_t stream);

}  // namespace mla
