// Triangle attention (starting node), forward and backward, for AMD gfx950 (MI355X).
//
// Method: "TurboPairFormer: Fast and Stable Protein Folding Model Training with an
// Optimized Triangle Attention Kernel" (arXiv 2610.05854), Abstract.  Per batch b,
// slice i and head h:  o[j] = sum_k softmax_k(alpha q[j].k[k] + bias[j,k] + m[k]) v[k],
// with the pair bias shared across all slices.  The backward is key-tile parallel: each
// probability tile is recomputed once and feeds all four gradients; dq (a sum over key
// blocks) and dbias (a sum over slices) go through ordered partial buffers, so there
// are no floating-point atomics and the results are bitwise reproducible.  The
// forward stores a bf16 copy of the output-rounding residual so that the softmax
// backward correction D = rowsum(dO * o) can be formed in FP32 (output-residual
// compensation, same Abstract).
//
// Hardware mapping (gfx950):
//  * QK^T and PV (and the five backward products) run on v_mfma_f32_32x32x16_bf16 /
//    v_mfma_f32_16x16x32_bf16 with FP32 accumulation.
//  * Operands whose contraction index is the token index (V in PV, Q/dO in dK/dV, K and
//    dS in dQ) are read from LDS with ds_read_b64_tr_b16, which hands each lane four
//    consecutive rows of one column.
//  * The pair bias is pre-scaled to FP32 (bias / alpha) in a tile order that matches the
//    MFMA accumulator layout, and is loaded straight into the accumulator before the
//    QK^T product, so adding it costs no vector ALU work.  Padding rows/columns hold
//    -inf, which turns every out-of-range key or query into an exact zero probability.
//  * Work-groups are numbered so that consecutive ids land on the same XCD (dispatch is
//    round-robin over the 8 XCDs), keeping one head's bias and the tiles shared by
//    neighbouring work-groups in that XCD's L2.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>
#include <math.h>

#include <mutex>
#include <type_traits>

#include "tri_attn.h"

namespace {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
// Largest finite fp16 magnitude: finite bias values are clamped to [-kBiasMax, kBiasMax] in both
// passes (the backward streams the bias as fp16), so forward and backward see the same scores.
constexpr float kBiasMax = 65504.0f;
constexpr int kXcd = 8;            // XCDs per MI355X; dispatch is round-robin over them

// Element offsets of the token tensors (q, k, v, o, residual, dO, dq, dk, dv): entry
// (b, i, h, j, c) of slice i, head h, token j, channel c sits at b*sB + i*sI + h*sH + j*sT + c.
// Channels are contiguous; a token row is D elements.
struct TokLayout {
  int64_t sB, sI, sH;
  int sT;
  __device__ __forceinline__ int64_t slice(int b, int i, int h) const {
    return (int64_t)b * sB + (int64_t)i * sI + (int64_t)h * sH;
  }
  // bytes spanned by the N token rows of one slice-head (what a buffer descriptor covers)
  __device__ __forceinline__ int span_bytes(int N, int D) const { return ((N - 1) * sT + D) * 2; }
};
// The kernels take a STRIDED flag: without it they use the slice-major layout [B, N, H, N, D]
// built here from the shape, so that its strides are compile-time multiples of D.
template <bool STRIDED, int D>
__device__ __forceinline__ TokLayout tok_layout(const TokLayout& given, int N, int H) {
  if (STRIDED) return given;
  return TokLayout{(int64_t)N * H * N * D, (int64_t)H * N * D, (int64_t)N * D, D};
}

// ------------------------------------------------------------------ small helpers

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 zero8() {
  bf16x8 z;
#pragma unroll
  for (int i = 0; i < 8; i++) z[i] = (bf16)0.0f;
  return z;
}

typedef __attribute__((address_space(3))) bf16 lbf16;
typedef __attribute__((address_space(3))) float lf32;
typedef __attribute__((address_space(3))) bf16x8 lbf16x8;
typedef __attribute__((address_space(3))) bf16x4 lbf16x4;
typedef __attribute__((address_space(3))) f32x4 lf32x4;
typedef __attribute__((address_space(3))) s16x4 ls16x4;
typedef unsigned u32x4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) u32x4v lu32x4;
typedef unsigned u32x2v __attribute__((ext_vector_type(2)));

// 32x32 product over k = 8 from two-dword operands (lane l: row or column l % 32, k = 4 (l / 32)
// + 0..3); as fast as the k = 16 form, with half the operand registers
typedef short s16x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x16 mfma32k8(u32x2v a, u32x2v b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(__builtin_bit_cast(s16x4v, a), __builtin_bit_cast(s16x4v, b), c, 0, 0, 0);
}

// x as three bf16 parts (hi, mid, lo: each the round-to-nearest-even of what the parts before it
// leave) and a zero, packed into two dwords; the parts sum to x exactly for a finite x below the
// bf16 range limit (24 significand bits in three 8-bit parts)
__device__ __forceinline__ u32x2v split3_bf16(float x) {
  const bf16 hi = (bf16)x;
  const float r1 = x - (float)hi;
  const bf16 mid = (bf16)r1;
  const bf16 lo = (bf16)(r1 - (float)mid);
  return u32x2v{(unsigned)__builtin_bit_cast(unsigned short, hi) | ((unsigned)__builtin_bit_cast(unsigned short, mid) << 16),
                (unsigned)__builtin_bit_cast(unsigned short, lo)};
}

// Lane part of a transposed read: lane t of a 16-lane group addresses row t/4 and
// column 4*(t%4) of the 4x16 block it helps to load.
__device__ __forceinline__ int tr_lane(int ld) {
  const int t = threadIdx.x & 15;
  return (t >> 2) * ld + 4 * (t & 3);
}
// ds_read_b64_tr_b16 at an LDS address that already contains the lane part: with
// p = &X[r0][c0] + tr_lane(ld), lane t of each 16-lane group receives X[r0+e][c0+t], e = 0..3.
__device__ __forceinline__ s16x4 tr16p(const lbf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((ls16x4*)p);
}

// Transposed LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes, lane t
// receives X[r0 + e][c0 + t] for e = 0..3, where X is a row-major bf16 matrix in LDS
// with leading dimension ld (elements).  r0, c0 must be uniform over the 16-lane group.
__device__ __forceinline__ s16x4 tr16(const bf16* X, int ld, int r0, int c0) {
  const int t = threadIdx.x & 15;
  const bf16* p = X + (r0 + (t >> 2)) * ld + c0 + 4 * (t & 3);
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
}
__device__ __forceinline__ bf16x8 cat8(s16x4 a, s16x4 b) {
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ bf16x8 pack8(const float* f) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; i++) r[i] = (bf16)f[i];
  return r;
}

// Work-group id -> logical tile, so that tiles [x*per, (x+1)*per) run on XCD x.
__device__ __forceinline__ int64_t xcd_tile(int64_t ntiles) {
  const int64_t per = (ntiles + kXcd - 1) / kXcd;
  return (int64_t)(blockIdx.x % kXcd) * per + blockIdx.x / kXcd;
}

__host__ __device__ constexpr int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// Offset of element (m, n) inside a 32x32 FP32 tile stored in "accumulator order":
// lane n%32 of lane-group g reads 16 contiguous bytes holding rows 8R+4g+0..3.
__host__ __device__ __forceinline__ int64_t ctile_off(int m, int n) {
  const int R = m >> 3, g = (m >> 2) & 1, e = m & 3;
  return ((int64_t)((R * 2 + g) * 32 + n)) * 4 + e;
}

// ------------------------------------------------------------------ bias preparation
// biasF: forward operand, 32x32 tiles indexed (b,h, query block, key block), element
// (row m = key k%32, column n = query j%32) in accumulator order; value bias[b,h,j,k]/alpha
// (finite values clamped to +-kBiasMax first, infinities kept), -inf for k >= N, 0 for padded
// queries j >= N.
__device__ __forceinline__ void bias_prep_fwd_elem(const bf16* __restrict__ bias, float* __restrict__ out, int N,
                                                   int Jp, int Kp, float inv_alpha, int64_t idx) {
  const int64_t tile = idx >> 10;
  const int off = (int)(idx & 1023);
  const int e = off & 3, n = (off >> 2) & 31, Rg = off >> 7;  // Rg = R*2+g
  const int m = (Rg >> 1) * 8 + (Rg & 1) * 4 + e;
  const int ncb = Kp / 32, nrb = Jp / 32;
  const int cb = (int)(tile % ncb);
  const int rb = (int)((tile / ncb) % nrb);
  const int64_t bh = tile / ((int64_t)ncb * nrb);
  const int j = rb * 32 + n, k = cb * 32 + m;
  float val;
  if (k >= N) val = -INFINITY;
  else if (j >= N) val = 0.0f;
  else {
    val = (float)bias[(bh * N + j) * N + k];
    if (!__builtin_isinf(val)) val = fminf(fmaxf(val, -kBiasMax), kBiasMax);
    val *= inv_alpha;
  }
  out[idx] = val;
}
__global__ void bias_prep_fwd_kernel(const bf16* __restrict__ bias, float* __restrict__ out, int N, int Jp, int Kp,
                                     float inv_alpha, int64_t total) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx < total) bias_prep_fwd_elem(bias, out, N, Jp, Kp, inv_alpha, idx);
}

// biasB: backward operand, fp16, one contiguous block per (b, h, 64-key block kb) that the
// backward work-group streams into LDS step by step.  Inside a block: 128-query step s, then
// tile t = 4*kh + p (key half kh, 32-query tile p), then 1024 values in lane order
// [half hf][lane 32g+n][8]: position 4R'+e of the 8 holds query 128s + 32p + 8(2hf+R') + 4g + e
// and key 64kb + 32kh + n, i.e. accumulator register 8hf+4R'+e of lane 32g+n of the 32x32
// score tile.  fp16 holds every bf16 value of magnitude 2^-17..65504 exactly (smaller ones
// to 2^-25 absolute); larger magnitudes saturate at 65504, infinities stay infinite, and the
// padding (j >= N or k >= N) is -inf.  The main kernel widens it inside v_fma_mix_f32.
__device__ __forceinline__ void bias_prep_bwd_elem(const bf16* __restrict__ bias, _Float16* __restrict__ out, int N,
                                                   int KB, int nsteps, int64_t idx) {
  const int off = (int)(idx & 1023), t = (int)((idx >> 10) & 7);
  int64_t rest = idx >> 13;
  const int s = (int)(rest % nsteps); rest /= nsteps;
  const int kb = (int)(rest % KB);
  const int64_t bh = rest / KB;
  const int e = off & 3, R = ((off >> 9) << 1) | ((off >> 2) & 1), lane = (off >> 3) & 63;
  const int j = s * 128 + (t & 3) * 32 + R * 8 + (lane >> 5) * 4 + e;
  const int k = kb * 64 + (t >> 2) * 32 + (lane & 31);
  float x = -INFINITY;
  if (j < N && k < N) {
    x = (float)bias[(bh * N + j) * N + k];
    if (!__builtin_isinf(x)) x = fminf(fmaxf(x, -kBiasMax), kBiasMax);
  }
  out[idx] = (_Float16)x;
}

// Both backward operands in one launch (they have the same element count, B*H*Kp*Jp): the
// backward's fp16 column blocks and, for its dQ kernel, the forward's FP32 tiles.
__global__ void bias_prep_bwd_kernel(const bf16* __restrict__ bias, _Float16* __restrict__ outB,
                                     float* __restrict__ outF, int N, int Jp, int Kp, int KB, int nsteps,
                                     float inv_alpha, int64_t total) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  bias_prep_bwd_elem(bias, outB, N, KB, nsteps, idx);
  bias_prep_fwd_elem(bias, outF, N, Jp, Kp, inv_alpha, idx);
}

// ------------------------------------------------------------------ streaming helpers

// Raw buffer resources (raw_rsrc below) cover [base, base + bytes): loads past the end return
// zeros, which is how rows beyond N are read.  The range check applies to the per-lane and the scalar
// offset together (a load at voffset + soffset >= bytes returns zeros; measured on gfx950 with
// every address inside the allocation), so row offsets may go into either.  (Only loads go through buffer resources: the compiler's
// wait-state rule for the store-data hazard of wide buffer stores does not cover the form
// with a register scalar offset on gfx950, where such stores were seen to write
// overwritten data.  Global stores get the wait states.)

// Direct-to-LDS loads written as inline assembly.  The compiler's own form of these loads
// makes it wait for every outstanding one before any later LDS read it cannot prove
// unrelated (the transposing reads among them), which would expose the latency of a
// prefetch issued one item ahead.  In this form the loads are invisible to the compiler's
// wait-count tracking; the kernels wait for them explicitly (vmcnt) before the barrier that
// publishes the data.  rsrc is a raw buffer descriptor (wave-uniform): base address, byte
// count (reads at or past it return zeros), raw flags.  The compiler does not look inside
// the statement for hazards, so it carries its own wait states: one between the write of
// M0 and the load that reads it, and five before a load whose scalar operands a vector
// instruction (readfirstlane, readlane) may have just written; s_nop 4 after the M0 write
// gives six.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 raw_rsrc(const void* base, int bytes) {
  const unsigned long long a = (unsigned long long)(uintptr_t)base;
  i32x4 r = {__builtin_amdgcn_readfirstlane((int)(unsigned)a),
             __builtin_amdgcn_readfirstlane((int)((unsigned)(a >> 32) & 0xFFFFu)),
             __builtin_amdgcn_readfirstlane(bytes), 0x00020000};
  return r;
}
__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return (unsigned)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}
// 16 bytes per lane: lane l's bytes land at LDS byte address lds_wave_base + 16 l
__device__ __forceinline__ void dma16_asm(i32x4 rsrc, unsigned voff, int soff, unsigned lds_wave_base) {
  asm volatile("s_mov_b32 m0, %3\n\ts_nop 4\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :: "v"(voff), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(soff)),
                  "s"(__builtin_amdgcn_readfirstlane(lds_wave_base)) : "memory", "m0");
}
__device__ __forceinline__ void dma16_asm(i32x4 rsrc, unsigned voff, int soff, const void* lds_wave_base) {
  dma16_asm(rsrc, voff, soff, lds_addr(lds_wave_base));
}
// as dma16_asm, issued only once `after` has been computed (an operand the statement ignores)
__device__ __forceinline__ void dma16_asm_after(i32x4 rsrc, unsigned voff, int soff, unsigned lds_wave_base, float after) {
  asm volatile("s_mov_b32 m0, %3\n\ts_nop 4\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :: "v"(voff), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(soff)),
                  "s"(__builtin_amdgcn_readfirstlane(lds_wave_base)), "v"(after) : "memory", "m0");
}
// one byte per lane, zero-extended into lane l's dword at LDS byte address lds_wave_base + 4 l
__device__ __forceinline__ void dma1_asm(i32x4 rsrc, unsigned voff, int soff, unsigned lds_wave_base) {
  asm volatile("s_mov_b32 m0, %3\n\ts_nop 4\n\tbuffer_load_ubyte %0, %1, %2 offen lds"
               :: "v"(voff), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(soff)),
                  "s"(__builtin_amdgcn_readfirstlane(lds_wave_base)) : "memory", "m0");
}

// fma(float(h), c, x) for the low (SEL = 0) or high (SEL = 1) fp16 half h of `pair`, in one
// v_fma_mix_f32 (the fp16 operand is widened exactly inside the instruction).  Its operands
// must come from memory loads or ordinary vector instructions, never straight from a
// matrix product: the compiler does not insert the wait states a product's result needs
// before an inline assembly statement reads it.
template <int SEL>
__device__ __forceinline__ float fma_mix_f16(unsigned pair, float c, float x) {
  float r;
  if (SEL == 0)
    asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[0,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(pair), "v"(c), "v"(x));
  else
    asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(pair), "v"(c), "v"(x));
  return r;
}

// Non-temporal (streaming) 16-byte global load: data read once per pass, kept out of the way
// of the tiles that are re-read.  (Streaming stores of partial lines measured slower.)
__device__ __forceinline__ bf16x8 ld_nt(const bf16x8* p) {
  return __builtin_bit_cast(bf16x8, __builtin_nontemporal_load((const u32x4v*)p));
}

// This lane's index in its wave, from a statement the compiler cannot move: a per-lane offset
// derived from it is recomputed where it is used instead of holding a register (or a spill
// slot) across a loop.  (Plain vector instructions, no hazard with the matrix products.)
__device__ __forceinline__ int lane_here() {
  int r;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(r));
  return r;
}

// Work-group barrier that orders LDS accesses only.  __syncthreads() also waits for every
// outstanding global access of the wave (its release fence covers the direct-to-LDS loads),
// which would expose the latency of a prefetch issued just before it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_sched_barrier(0);   // no instruction moves across (register pressure)
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
}

// chunk swizzle for rows of D bf16 (D/8 chunks of 16 bytes per row)
template <int D>
__device__ __forceinline__ int swz(int row) {
  return D == 32 ? ((row >> 2) & 3) : ((row >> 3) & 1);
}

// Element offset, in a row-swizzled [rows][D] bf16 tile, of the 8 bytes this lane reads for a
// transposed load of the 4-row group starting at r0 (column block c0, 16 columns).
template <int D>
__device__ __forceinline__ int tr_off(int lane, int r0, int c0) {
  const int t16 = lane & 15;
  const int rr = r0 + (t16 >> 2), col = c0 + 4 * (t16 & 3);
  return rr * D + ((((col >> 3) ^ swz<D>(rr)) << 3) | (col & 7));
}

// ------------------------------------------------------------------ forward
// One work-group = 4 waves = 128 queries of one slice (b,i,h); wave w owns 32 queries.
// S^T (keys x queries) = K Q^T on 32x32x16 MFMA: each lane holds one query column and
// 16 keys per 32-key tile, so the running max/sum of a query needs one cross-lane step.
// The accumulator of each score tile starts from the prepared bias/alpha tile.
//
// Software pipeline over 64-key tiles: while tile t's softmax and PV product run, tile t+1's
// K and V (shared by the work-group) stream into the other half of double-buffered LDS
// (direct-to-LDS loads, issued once tile t's scores are complete); keys past N read as zeros.
// Each wave reads its two bias tiles of tile t straight from global memory into the score
// accumulators (every slice of a head reads the same tiles, so they come from L2), issued
// before the barrier that publishes tile t so that their latency overlaps that wait; padded
// keys carry a -inf bias.  K and V rows are XOR-swizzled like the backward's.
// (five waves per SIMD; the d = 32 instances with a key mask or strided rows need the registers of
// four to run without spilling, which measured as fast or faster)
template <int D, bool MASK, bool STRIDED>
__global__ __launch_bounds__(256, D == 32 && (MASK || STRIDED) ? 4 : 5)
void fwd_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
                const float* __restrict__ biasF, const uint8_t* __restrict__ mask,
                bf16* __restrict__ o, float* __restrict__ lse, bf16* __restrict__ res,
                int B, int N, int H, float alpha, TokLayout Lg) {
  const TokLayout L = tok_layout<STRIDED, D>(Lg, N, H);
  constexpr int KT = 64;        // keys per iteration
  constexpr int NC = D / 16;    // 16-wide channel chunks
  constexpr int CPR = D / 8;    // 16-byte chunks per row
  __shared__ __attribute__((aligned(16))) bf16 Ks_[2][KT * D];
  __shared__ __attribute__((aligned(16))) bf16 Vs_[2][KT * D];
  __shared__ __attribute__((aligned(16))) uint8_t Ms_[2][KT];
  // D = 16: a tile of ones read in place of V by the lanes of the product's upper 16 rows
  __shared__ __attribute__((aligned(16))) bf16 Ones_[D == 16 ? KT * 16 : 8];

  const int QT = (N + 127) / 128;
  const int64_t ntiles = (int64_t)B * H * N * QT;
  const int64_t tile = xcd_tile(ntiles);
  if (tile >= ntiles) return;
  // Tile order: query tiles fastest, then slices, then heads, so that the work-groups on one
  // XCD share one head's prepared bias tiles in its L2 (also in the strided layouts, where
  // putting the heads first was measured 1.7x slower: the bias tiles of all heads no longer fit).
  const int qt = (int)(tile % QT);
  int64_t rest = tile / QT;
  const int i = (int)(rest % N); rest /= N;
  const int h = (int)(rest % H);
  const int b = (int)(rest / H);

  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, g = l >> 5, ln = l & 31;
  const int64_t sbase = L.slice(b, i, h);
  const int sT = L.sT;
  const int j = qt * 128 + w * 32 + ln;  // this lane's query
  const bool jok = j < N;
  const int Kp = (int)round_up(N, 64), Jp = (int)round_up(N, 128);
  const float* btile = biasF + ((int64_t)(b * H + h) * (Jp / 32) + (qt * 4 + w)) * (int64_t)(Kp / 32) * 1024;
  const float c1 = alpha * kLog2e;
  const uint8_t* mrow = MASK ? mask + ((int64_t)b * N + i) * N : nullptr;

  // streamed loads: K and V rows (lane -> swizzled 16-byte chunk), this wave's bias tiles
  // (inline-assembly loads, which the compiler's own waits do not cover: see dma16_asm)
  const i32x4 rk = raw_rsrc(k + sbase, L.span_bytes(N, D)), rv = raw_rsrc(v + sbase, L.span_bytes(N, D));
  const unsigned kv_vo = (unsigned)(((tid / CPR) * sT + ((tid % CPR) ^ swz<D>(tid / CPR)) * 8) * 2);
  auto prefetch = [&](int kt, int buf, float after) {
    if (w < KT * CPR / 64) {
      dma16_asm_after(rk, kv_vo, kt * KT * sT * 2, lds_addr(&Ks_[buf][w * 512]), after);
      dma16_asm_after(rv, kv_vo, kt * KT * sT * 2, lds_addr(&Vs_[buf][w * 512]), after);
    }
  };

  bf16x8 qf[NC];
#pragma unroll
  for (int cc = 0; cc < NC; cc++)
    qf[cc] = jok ? *(const bf16x8*)(q + sbase + (int64_t)j * sT + cc * 16 + g * 8) : zero8();

  f32x16 acc_o = {};
  float m_run = -INFINITY, l_run = 0.0f;
  // D = 32: the sum of the bf16 probabilities that multiply V, through one 16x16x32 product per
  // PV product (A: ones in row 0 at the k groups of query n, row 1 at those of query n + 16);
  // lanes 0-15 hold it for queries l and l + 16 in registers 0 and 1
  f32x4 psum = {};
  const int lm = l & 15, lk = l >> 4;
  const bool onesA = (lm == 0 && (lk & 1) == 0) || (lm == 1 && (lk & 1) == 1);
  const unsigned oa = onesA ? 0x3F803F80u : 0u;
  const bf16x8 oneA = __builtin_bit_cast(bf16x8, u32x4v{oa, oa, oa, oa});

  const int nkt = (N + KT - 1) / KT;
  if (MASK && tid < KT) Ms_[0][tid] = tid < N ? mrow[tid] : (uint8_t)1;
  if (D == 16) ((__attribute__((address_space(3))) u32x2v*)Ones_)[tid] = u32x2v{0x3F803F80u, 0x3F803F80u};  // read after the first barrier
  prefetch(0, 0, 0.0f);
  // Key tile kt in LDS buffer CUR.  The buffer index is a compile-time constant (the loop below
  // runs two tiles per pass), so every LDS address is a per-lane offset plus an immediate.
  auto key_tile = [&](int kt, auto cur_) {
    constexpr int cur = decltype(cur_)::value;
    // this wave's bias tiles of tile kt: eight 16-byte loads into the score accumulators
    f32x16 s[2];
#pragma unroll
    for (int tt = 0; tt < 2; tt++) {
#pragma unroll
      for (int R = 0; R < 4; R++) {
        const f32x4 bv = *(const f32x4*)(btile + (int64_t)(kt * 2 + tt) * 1024 + ((R * 2 + g) * 32 + ln) * 4);
        s[tt][R * 4 + 0] = bv[0]; s[tt][R * 4 + 1] = bv[1];
        s[tt][R * 4 + 2] = bv[2]; s[tt][R * 4 + 3] = bv[3];
      }
    }
    // every load but those eight, among them this wave's part of tile kt, has landed (loads
    // complete in issue order; the memory clobber keeps the bias loads above the wait)
    asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    __syncthreads();  // all of tile kt is in LDS; buffer cur^1 is free
    uint8_t mnext = 1;
    if (MASK && kt + 1 < nkt && tid < KT && (kt + 1) * KT + tid < N) mnext = mrow[(kt + 1) * KT + tid];
    const lbf16* Ks = (const lbf16*)Ks_[cur];
    const lbf16* Vs = (const lbf16*)Vs_[cur];

#pragma unroll
    for (int tt = 0; tt < 2; tt++) {
      const int rk_ = tt * 32 + ln;
#pragma unroll
      for (int cc = 0; cc < NC; cc++) {
        const bf16x8 a = *(const lbf16x8*)(Ks + rk_ * D + ((cc * 2 + g) ^ swz<D>(rk_)) * 8);
        s[tt] = mfma32(a, qf[cc], s[tt]);
      }
      if (MASK) {
        // a masked key's row of S^T gets -2^100 through one k = 8 product (A: -2^100 at k = 0 of
        // the lane's key row rk_, B: one at k = 0; a kept key's row gets an exact 0): once a kept
        // key has set the reference its probability is exactly zero, and a row whose maximum stays
        // below -2^99 has no kept key (epilogue)
        const u32x2v mA = {(g == 0 && !Ms_[cur][rk_]) ? 0xF180u : 0u, 0u};
        s[tt] = mfma32k8(mA, u32x2v{g == 0 ? 0x3F80u : 0u, 0u}, s[tt]);
      }
    }
    // maximum over this lane's 32 scores (NaN-propagating maximum: three-operand instructions
    // with no quieting of the matrix products' results)
    float mx = __builtin_elementwise_maximum(s[0][0], s[0][1]);
#pragma unroll
    for (int r = 2; r < 16; r += 2)
      mx = __builtin_elementwise_maximum(__builtin_elementwise_maximum(mx, s[0][r]), s[0][r + 1]);
#pragma unroll
    for (int r = 0; r < 16; r += 2)
      mx = __builtin_elementwise_maximum(__builtin_elementwise_maximum(mx, s[1][r]), s[1][r + 1]);
    // the next tile's K and V, issued once this tile's scores exist: the compiler's waits for
    // the bias loads then never include them, and they stream during the softmax and PV
    if (kt + 1 < nkt) prefetch(kt + 1, cur ^ 1, mx);
    // The reference maximum of a query moves only when a score exceeds it by more than
    // 2^8 in probability (exp2 units): probabilities stay <= 256, exact in FP32 and with
    // bf16's relative precision, and most tiles skip the rescale of the accumulators.  The
    // tests are written so that a NaN comparison counts as growth.  A query's scores are split
    // over the lane pair (l, l^32): the pair's maximum exceeds the bound only if one lane's does,
    // so the exchange between the two lanes happens only when some lane of the wave sees
    // growth (a wave-uniform branch, all lanes active for the exchange).
    if (__builtin_amdgcn_ballot_w64(!(mx * c1 <= m_run * c1 + 8.0f))) {
      mx = __builtin_elementwise_maximum(mx, __shfl_xor(mx, 32));
      const bool grow = !(mx * c1 <= m_run * c1 + 8.0f);
      const float m_new = grow ? fmaxf(m_run, mx) : m_run;
      const float scale = grow ? __builtin_amdgcn_exp2f((m_run - m_new) * c1) : 1.0f;
      m_run = m_new;
      l_run *= scale;
#pragma unroll
      for (int r = 0; r < 16; r++) acc_o[r] *= scale;
      if (D == 32) {
        const float s16 = __shfl(scale, lm + 16);
        psum[0] *= scale;
        psum[1] *= s16;
      }
    }
    // (while every score so far is -inf, the reference is 0: exp2(-inf - 0) = 0, not NaN)
    const float nm = m_run == -INFINITY ? 0.0f : m_run * c1;
    float p[2][16];
    float lsum = 0.0f;
#pragma unroll
    for (int tt = 0; tt < 2; tt++)
#pragma unroll
      for (int r = 0; r < 16; r++) {
        p[tt][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[tt][r], c1, -nm));
        lsum += p[tt][r];
      }
    l_run += lsum;

    // O^T (channels x queries) += V^T P^T; lane group (l/16) selects channel half and key run.
    // At D = 16 the lanes of the upper 16 rows read ones: those rows accumulate the sum of the
    // bf16 probabilities that multiply V, which normalises o (the FP32 sum gives lse).
    const int G16 = l >> 4, chalf = G16 & 1;
    const lbf16* Va = (D == 16 && chalf) ? (const lbf16*)Ones_ : Vs;
#pragma unroll
    for (int tt = 0; tt < 2; tt++)
#pragma unroll
      for (int m2 = 0; m2 < 2; m2++) {
        const bf16x8 pb = pack8(&p[tt][m2 * 8]);
        const int r0 = tt * 32 + m2 * 16 + g * 4;
        const int c0 = D == 32 ? chalf * 16 : 0;
        const bf16x8 a = cat8(tr16p(Va + tr_off<D>(l, r0, c0)), tr16p(Va + tr_off<D>(l, r0 + 8, c0)));
        acc_o = mfma32(a, pb, acc_o);
        if (D == 32) psum = mfma16(oneA, pb, psum);
      }
    if (MASK && tid < KT) Ms_[cur ^ 1][tid] = mnext;  // read after the next barrier
  };
  for (int kt = 0; kt < nkt; kt += 2) {
    key_tile(kt, std::integral_constant<int, 0>{});
    if (kt + 1 < nkt) key_tile(kt + 1, std::integral_constant<int, 1>{});
  }

  // epilogue: normalise, round, residual, logsumexp.  A query with no key of finite score (every
  // key masked, or every key's bias -inf) attends to nothing: o = 0, residual 0, lse = +inf, which
  // gives every one of its probabilities in the backward exp(s - lse) = 0.  (With every key masked
  // the reference maximum is about -2^100, far below any score of a kept key.)
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const bool empty = !(l_tot > 0.0f) || (MASK && !(m_run > -0x1p99f));
  // o is normalised by the sum of the probabilities as they entered the product (D = 16: an
  // upper row of the product; every kept row has one probability >= 1 there)
  const float plo = __shfl(psum[0], ln & 15), phi = __shfl(psum[1], ln & 15);
  const float inv = empty ? 0.0f : 1.0f / (D == 16 ? acc_o[8] : (ln < 16 ? plo : phi));
  if (jok) {
    bf16* orow = o + sbase + (int64_t)j * sT;
    bf16* rrow = res ? res + sbase + (int64_t)j * sT : nullptr;
#pragma unroll
    for (int R = 0; R < D / 8; R++) {
      bf16x4 ob, rb;
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const float f = acc_o[R * 4 + e] * inv;
        const bf16 fb = (bf16)f;
        ob[e] = fb;
        rb[e] = (bf16)(f - (float)fb);
      }
      const int c = R * 8 + g * 4;
      *(bf16x4*)(orow + c) = ob;
      if (rrow) *(bf16x4*)(rrow + c) = rb;
    }
    if (g == 0) lse[(((int64_t)b * N + i) * H + h) * N + j] = empty ? INFINITY : m_run * alpha + logf(l_tot);
  }
}

// ------------------------------------------------------------------ backward: main
// One work-group = 8 waves = one block of 64 keys of head h, for a group of G slices.
// wave w: key half kh = w&1 (32 keys), query lane p = w>>1.  The work items are
// (slice, 128-query step) pairs; step s of a slice covers queries 128s..128s+127 in four
// tiles of 32, tile p going to query lane p.  Each wave keeps the pair-bias gradient of
// its (query tiles x 32 keys) in registers across the slice group ("face"), so dS is
// summed over slices on chip and written once per group.  The steps of a slice are
// unrolled at compile time so that every face slot is addressed statically.
//
// dQ is not formed here: it sums over every key block, and dq_kernel computes it on its own
// (see there), so nothing leaves this work-group but dK, dV and the pair-bias gradient.
//
// Software pipeline: while item t is computed, each wave's own part of item t+1 (its 32 Q and dO
// rows, its pair-bias tile and its queries' row statistics) streams from global memory straight
// into the other half of the wave's private double buffer in LDS (direct-to-LDS loads, no
// registers involved; each wave waits for its own loads), and the next slice's K, V and
// key-mask bytes stream into the other of two shared K/V buffers from the first item of a slice
// on.  The work-group meets at two barriers per slice: at its start (the slice's K/V are in LDS
// and no wave reads the previous slice's any more) and in the dK/dV reduction at its end.  Rows
// past N read as zeros through the buffer range check, and the -inf padding of the prepared bias
// turns every padded query or key into an exact zero probability.
//
// Rows of Q, dO, K and V in LDS hold their 16-byte chunks in XOR-swizzled order (chunk c
// of row r sits in slot c ^ swz(r)), which spreads the row-wise operand reads of a wave
// over all LDS banks.
constexpr int kBwdMaxSteps = 6;  // 128-query steps of one work-group (768 queries)

// s_waitcnt vmcnt(n) for a wave-uniform n in 0..15 (the instruction takes an immediate)
__device__ __forceinline__ void wait_vmcnt(int n) {
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    case 1: __builtin_amdgcn_s_waitcnt(0x0F71); break;
    case 2: __builtin_amdgcn_s_waitcnt(0x0F72); break;
    case 3: __builtin_amdgcn_s_waitcnt(0x0F73); break;
    case 4: __builtin_amdgcn_s_waitcnt(0x0F74); break;
    case 5: __builtin_amdgcn_s_waitcnt(0x0F75); break;
    case 6: __builtin_amdgcn_s_waitcnt(0x0F76); break;
    case 7: __builtin_amdgcn_s_waitcnt(0x0F77); break;
    case 8: __builtin_amdgcn_s_waitcnt(0x0F78); break;
    case 9: __builtin_amdgcn_s_waitcnt(0x0F79); break;
    case 10: __builtin_amdgcn_s_waitcnt(0x0F7A); break;
    case 11: __builtin_amdgcn_s_waitcnt(0x0F7B); break;
    case 12: __builtin_amdgcn_s_waitcnt(0x0F7C); break;
    case 13: __builtin_amdgcn_s_waitcnt(0x0F7D); break;
    case 14: __builtin_amdgcn_s_waitcnt(0x0F7E); break;
    default: __builtin_amdgcn_s_waitcnt(0x0F7F); break;
  }
}

// Query chunks of the backward for N past six 128-query steps: a work-group keeps the pair-bias
// gradient of its chunk's queries in registers (at most six steps), so longer slices are split
// into ceil(steps / 6) chunks as equal as possible (cs or cs - 1 steps), each its own set of
// work-groups, in one launch per chunk length.  dQ rows and dbias rows of different chunks are
// disjoint; dK and dV sum over all queries, so chunked work-groups write FP32 partials per
// chunk, summed in chunk order by reduce_dkv_kernel.
struct Chunking {
  int nst;       // 128-query steps per slice in total
  int c_begin;   // first chunk of this launch (all of whose chunks have NS steps)
  int ncl;       // chunks in this launch
  int step0;     // first 128-query step of this launch's first chunk
  float* dkvp;   // FP32 partials [chunk][dk, dv][B*N*H slice-head rows][N keys][D]
};

template <int D, bool MASK, int NS, bool STRIDED, bool CHUNKED>
__global__ __launch_bounds__(512, 1)
void bwd_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
                const bf16* __restrict__ dO, const bf16* __restrict__ biasB, const uint8_t* __restrict__ mask,
                const unsigned* __restrict__ LDp, float* __restrict__ dbp, bf16* __restrict__ dk, bf16* __restrict__ dv,
                int B, int N, int H, int G, int ngroups, float alpha, TokLayout Lg, Chunking Ck) {
  const TokLayout L = tok_layout<STRIDED, D>(Lg, N, H);
  constexpr int NC = D / 16;
  constexpr int CPR = D / 8;    // 16-byte chunks per row
  constexpr int NR = D / 2;     // accumulator registers of dK^T / dV^T holding channels c < D
  // LDS map (bytes): per wave, two item buffers of [its 32 Q rows | its 32 dO rows | its 32x32
  // pair-bias tile | its 32 queries' row statistics, 16 bytes each] | K,V,mask x2 | dV reduction
  // (the waves' partials; their dK partials go to their own free item buffer)
  constexpr int kWQ = 32 * D * 2;                   // 32 rows of Q (or dO)
  constexpr int kWB = 2 * kWQ + 2048 + 512;         // one item buffer of one wave
  static_assert(NR * 64 * 4 <= kWB, "a wave's dK^T partial fits its item buffer");
  constexpr int kKVB = 2 * 64 * D * 2 + 64 * 4;     // K rows, V rows, 64 mask bytes (one per dword)
  // slice-end dK/dV sums shared by the four query lanes (D = 32), or made by the p = 0 lanes
  constexpr bool kShared = D == 32;
  constexpr int kWriters = kShared ? 4 : 3;         // waves per key half writing partials
  constexpr int kREDB = 2 * kWriters * NR * 64 * 4; // their dV^T partials
  constexpr int oKV = 8 * 2 * kWB, oRED = oKV + 2 * kKVB, kLdsBytes = oRED + kREDB;
  static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];

  const int KB = (N + 63) / 64;
  const int64_t per_chunk = (int64_t)B * H * ngroups * KB;
  const int64_t ntiles = CHUNKED ? per_chunk * Ck.ncl : per_chunk;
  const int64_t tile0 = xcd_tile(ntiles);
  if (tile0 >= ntiles) return;
  const int64_t tile = CHUNKED ? tile0 % per_chunk : tile0;
  const int chunk = CHUNKED ? Ck.c_begin + (int)(tile0 / per_chunk) : 0;
  // first 128-query step of this work-group's chunk
  const int s_base = CHUNKED ? Ck.step0 + (int)(tile0 / per_chunk) * NS : 0;
  const int NSt = CHUNKED ? Ck.nst : NS;    // 128-query steps per slice in total
  // Tile order: the key blocks of one (head, slice group) adjacent, so that they run together
  // on one XCD and share its L2 for the slices' Q and dO rows.  In a strided layout the heads
  // of one token row also share cache lines, so there the heads come fastest.
  int kb, grp, h, b;
  if (STRIDED) {
    h = (int)(tile % H);
    int64_t rest = tile / H;
    kb = (int)(rest % KB); rest /= KB;
    grp = (int)(rest % ngroups);
    b = (int)(rest / ngroups);
  } else {
    kb = (int)(tile % KB);
    int64_t rest = tile / KB;
    grp = (int)(rest % ngroups); rest /= ngroups;
    h = (int)(rest % H);
    b = (int)(rest / H);
  }
  const int i_begin = grp * G, i_end = min(N, i_begin + G);

  // the wave index is uniform; readfirstlane lets the compiler keep everything derived
  // from it (LDS destinations, tile offsets) in scalar registers
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, g = l >> 5, ln = l & 31;
  const int kh = w & 1, p = w >> 1;
  const int kl = kh * 32 + ln;          // key within the block
  const int kg = kb * 64 + kl;          // global key of this lane
  const bool kok = kg < N;
  // NS = ceil(N / 128) 128-query steps per slice, fixed at compile time so that the step
  // loop, its buffer parity (for even NS) and every step offset are constants
  constexpr int nsteps = NS;
  const int Jpt = NSt * 128;  // padded queries per slice (all chunks)
  const float c1 = alpha * kLog2e;
  const int sT = L.sT;
  const int span = L.span_bytes(N, D);                                   // bytes of a slice-head's rows

  // Per-lane byte offsets of the streamed loads of a wave's item, fixed for the whole work-group
  // (slice and step enter through the buffer base and the scalar offset): Q and dO rows p*32 + l/CPR
  // (+16 per further load at D = 32), which land swizzled like K and V; the row statistics of the
  // wave's 32 queries (lanes 0-31, one query each).
  const unsigned qd_vo = (unsigned)(((p * 32 + l / CPR) * sT + ((l % CPR) ^ swz<D>(l / CPR)) * 8) * 2);
  const unsigned ld_vo = (unsigned)((p * 32 + (l & 31)) * 16);
  const bf16* bias_blk = biasB + (((int64_t)(b * H + h) * KB + kb) * NSt + s_base) * (int64_t)8192;

  // Per-lane LDS byte offsets of the operand reads; the buffer and the step enter as uniform
  // additions or immediate offsets.
  //  * row reads (A/B operands of the 32x32x16 products): row ln of the wave's Q / dO rows or row
  //    kh*32 + ln of K / V, chunk cc*2+g in swizzled position; the swizzle depends on ln only
  //  * transposed reads of dO/Q (dV^T, dK^T A operands) over the wave's rows m2*16 + 4g (+8)
  const int swl = swz<D>(ln);
  unsigned offR[NC];
#pragma unroll
  for (int cc = 0; cc < NC; cc++) offR[cc] = (unsigned)((ln * D + (((cc * 2 + g) ^ swl) * 8)) * 2);
  const unsigned offK = (unsigned)(kh * 32 * D * 2);
  const int G16 = l >> 4, chalf = G16 & 1;
  const int c0 = D == 32 ? 16 * chalf : 0;
  const unsigned trA = (unsigned)(tr_off<D>(l, 4 * g, c0) * 2);
  const unsigned trB = (unsigned)(tr_off<D>(l, 4 * g + 8, c0) * 2);
  const unsigned offBias = (unsigned)(2 * kWQ + l * 16);
  const u32x2v one3 = g == 0 ? u32x2v{0x3F803F80u, 0x3F80u} : u32x2v{0u, 0u};  // ones at k = 0..2
  const unsigned offRow = (unsigned)(2 * kWQ + 2048 + ln * 16);  // row statistics of query row ln

  // issue the loads of work item (ii, ss) into LDS buffer `buf`; rows past N read as zeros
  // LDS byte address of the work-group's LDS block; the streamed loads take LDS addresses
  // relative to it and buffer descriptors built once per slice (the buffer range of a
  // slice-head row returns zeros for rows past N)
  const unsigned lds0 = __builtin_amdgcn_readfirstlane(lds_addr(lds));
  const i32x4 rbias = raw_rsrc(bias_blk, nsteps * 16384);  // this work-group's pair-bias column
  // per slice-head row: the descriptors of its Q, dO and row-statistics rows
  struct RowRes { i32x4 q, dO, ld; };
  auto row_res = [&](int ii) {
    const int64_t sl = ((int64_t)b * N + ii) * H + h;  // slice-head row index
    RowRes r;
    const int64_t tb = L.slice(b, ii, h);
    r.q = raw_rsrc(q + tb, span);
    r.dO = raw_rsrc(dO + tb, span);
    r.ld = raw_rsrc(LDp + sl * 4 * Jpt, Jpt * 16);
    return r;
  };
  // issue the loads of this wave's part of work item (slice with row descriptors rr, step ss)
  // into its item buffer `buf`: everything a wave reads during an item but K and V comes from its
  // own loads, so that between the first items of two slices no wave waits for another
  auto prefetch = [&](const RowRes& rr, int ss, int buf) {
    const unsigned dst = lds0 + (unsigned)((w * 2 + buf) * kWB);
    const int so = (s_base + ss) * 128 * sT * 2;
#pragma unroll
    for (int m = 0; m < CPR / 2; m++) {  // 64 lanes x 16 bytes: 16 rows (D = 32) or 32 rows (D = 16)
      dma16_asm(rr.q, qd_vo, so + m * 16 * sT * 2, dst + m * 1024);
      dma16_asm(rr.dO, qd_vo, so + m * 16 * sT * 2, dst + kWQ + m * 1024);
    }
    // this wave's 32x32 pair-bias tile of the step (2 KiB)
    dma16_asm(rbias, (unsigned)l * 16u, ss * 16384 + (kh * 4 + p) * 2048, dst + 2 * kWQ);
    dma16_asm(rbias, (unsigned)l * 16u, ss * 16384 + (kh * 4 + p) * 2048 + 1024, dst + 2 * kWQ + 1024);
    if (l < 32) dma16_asm(rr.ld, ld_vo, (s_base + ss) * 2048, dst + 2 * kWQ + 2048);
  };
  // K, V and the key-mask bytes of slice ii into K/V buffer kvb
  auto prefetch_kv = [&](int ii, int kvb) {
    constexpr int KC = 64 * CPR;  // 16-byte chunks per block
    const int64_t tb = L.slice(b, ii, h);
    const unsigned dst = lds0 + oKV + kvb * kKVB;
    const int kv_t = (w & 3) * 64 + lane_here();  // K (waves 0-3) / V (waves 4-7); recomputed per slice
    const unsigned kv_vo = (unsigned)(((kb * 64 + kv_t / CPR) * sT + ((kv_t % CPR) ^ swz<D>(kv_t / CPR)) * 8) * 2);
    if (w < KC / 64) dma16_asm(raw_rsrc(k + tb, span), kv_vo, 0, dst + w * 1024);
    else if (w >= 4 && w < 4 + KC / 64)
      dma16_asm(raw_rsrc(v + tb, span), kv_vo, 0, dst + 64 * D * 2 + (w - 4) * 1024);
    if (MASK && w == 7)  // one byte per lane, each landing in its own dword
      dma1_asm(raw_rsrc(mask + ((int64_t)b * N + ii) * N, N), (unsigned)(kb * 64 + lane_here()), 0,
               dst + 2 * 64 * D * 2);
  };

  f32x16 face[NS];
#pragma unroll
  for (int s = 0; s < NS; s++) face[s] = f32x16{};

  prefetch_kv(i_begin, 0);
  RowRes rr_cur = row_res(i_begin);  // descriptors of slice i
  prefetch(rr_cur, 0, 0);

  // VMEM operations a wave issues after an item's prefetch and before that item's wait: after
  // the last item of a slice, its dK/dV stores (two per wave at D = 32; at D = 16 four, by the
  // p = 0 waves), made only by waves whose 32 keys are not all past N (the stores sit behind that
  // wave-uniform test, so each one the count includes is issued with at least one active lane)
  const bool any_key = kb * 64 + kh * 32 < N;
  const int kvStores = !any_key ? 0 : kShared ? 2 : (p == 0 ? 2 * (NR / 4) : 0);
  int ns_rt = NS;
  asm volatile("" : "+s"(ns_rt));
  int t = 0;        // item index within the work-group
  int cur_rt = 0;   // LDS buffer of item t (its parity)
  for (int i = i_begin; i < i_end; i++) {
    const int64_t sl_row = ((int64_t)b * N + i) * H + h;  // slice-head row index
    const int64_t sbase = L.slice(b, i, h);
    const int kvc = (i - i_begin) & 1;                     // K/V buffer of this slice
    const char* Ks = lds + oKV + kvc * kKVB;
    const char* Vs = Ks + 64 * D * 2;
    float mterm = 0.0f;
    f32x16 dkT = {}, dvT = {};
    const RowRes rr_next = row_res(min(i + 1, i_end - 1));  // descriptors of slice i+1
    // this wave's K and V rows of the slice (B operands of the two score products), read from
    // LDS at the slice's first item and held in registers for the rest of the slice
    bf16x8 kf[NC], vf[NC];

    auto step = [&](auto S_) {
      constexpr int s = decltype(S_)::value;
      // (a run-time value: with constant buffer offsets the compiler would keep a base
      // register per buffer and region live across the loop)
      const int cur = cur_rt;
      // wait for this wave's loads of item t (issued one item earlier); what follows them in the
      // queue is, at a slice start, the dK/dV stores
      if (t == 0) wait_vmcnt(0);
      else wait_vmcnt(s == 0 ? kvStores : 0);
      // at a slice start: the slice's K, V and mask bytes (loaded by all waves during the previous
      // slice) are in LDS everywhere, and no wave reads the previous slice's K/V buffer any more
      if (s == 0) lds_barrier();
      if (s == 0 && i + 1 < i_end) prefetch_kv(i + 1, (i + 1 - i_begin) & 1);
      {  // the next item: step s+1 of this slice, else step 0 of the next slice
        const bool same = s + 1 < nsteps;
        RowRes rn;
        rn.q = same ? rr_cur.q : rr_next.q;
        rn.dO = same ? rr_cur.dO : rr_next.dO;
        rn.ld = same ? rr_cur.ld : rr_next.ld;
        if (same || i + 1 < i_end) prefetch(rn, same ? s + 1 : 0, cur ^ 1);
      }
      if (MASK && s == 0) {
        const unsigned mb = *(const __attribute__((address_space(3))) unsigned*)(Ks + 2 * 64 * D * 2 + kl * 4);
        mterm = (kok && (mb & 0xFFu) == 0) ? -INFINITY : 0.0f;
      }

      const char* qd = lds + (w * 2 + cur) * kWB;  // this wave's item buffer: Q rows, dO rows, ...
      const char* ld = qd + offRow;

      // S - lse/alpha = Q K^T - lse/alpha (rows: 32 queries, cols: 32 keys) and dP - D = dO V^T - D.
      // The row terms enter through one k = 8 product each: A holds the three bf16 parts of the
      // row's value at k = 0..2 (lanes of the upper k half hold k = 4..7, multiplied by zeros of
      // B), B holds ones at k = 0..2.  The parts sum exactly to the FP32 value.
      f32x16 sacc, dp;
      // all operand reads of the two products are issued before the first product, so that
      // their latencies overlap instead of chaining read -> product -> read
      bf16x8 aq[NC], ao[NC];
#pragma unroll
      for (int cc = 0; cc < NC; cc++) {
        aq[cc] = *(const lbf16x8*)(qd + offR[cc]);
        if (s == 0) kf[cc] = *(const lbf16x8*)(Ks + offK + offR[cc]);
        ao[cc] = *(const lbf16x8*)(qd + kWQ + offR[cc]);
        if (s == 0) vf[cc] = *(const lbf16x8*)(Vs + offK + offR[cc]);
      }
      const u32x4v rs = *(const lu32x4*)ld;  // row statistics of this lane's query row
      __builtin_amdgcn_sched_barrier(0);
      sacc = mfma32k8(u32x2v{rs.x, rs.y}, one3, f32x16{});
      dp = mfma32k8(u32x2v{rs.z, rs.w}, one3, f32x16{});
#pragma unroll
      for (int cc = 0; cc < NC; cc++) {
        sacc = mfma32(aq[cc], kf[cc], sacc);
        dp = mfma32(ao[cc], vf[cc], dp);
      }

      // P = exp2(c1 (S - lse/alpha) + log2e bias) and dS = P (dP - D); dS is summed into the face.
      // The bias term is one v_fma_mix_f32 per element (fp16 bias pairs).
      const char* bS = qd + offBias;
      const u32x4v b0 = *(const lu32x4*)bS, b1 = *(const lu32x4*)(bS + 1024);
      float P[16], dS[16];
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const unsigned pr = r < 8 ? b0[(r & 7) >> 1] : b1[(r & 7) >> 1];
        const float t = sacc[r] * c1;
        float z = (r & 1) ? fma_mix_f16<1>(pr, kLog2e, t) : fma_mix_f16<0>(pr, kLog2e, t);
        if (MASK) z += mterm;
        P[r] = __builtin_amdgcn_exp2f(z);
        dS[r] = P[r] * dp[r];
      }
#pragma unroll
      for (int r = 0; r < 16; r++) face[s][r] += dS[r];

      // dV^T += dO^T P ; dK^T += Q^T dS   (rows: channels, cols: keys).  At D = 16 the upper
      // 16 channel rows of the 32x32 product repeat the lower ones and are never stored.
      bf16x8 pb[2], sb[2];
#pragma unroll
      for (int m2 = 0; m2 < 2; m2++) {
        pb[m2] = pack8(&P[m2 * 8]);
        sb[m2] = pack8(&dS[m2 * 8]);
      }
#pragma unroll
      for (int m2 = 0; m2 < 2; m2++) {
        const bf16x8 ao = cat8(tr16p((const lbf16*)(qd + kWQ + trA + m2 * 16 * D * 2)),
                               tr16p((const lbf16*)(qd + kWQ + trB + m2 * 16 * D * 2)));
        const bf16x8 aq = cat8(tr16p((const lbf16*)(qd + trA + m2 * 16 * D * 2)),
                               tr16p((const lbf16*)(qd + trB + m2 * 16 * D * 2)));
        dvT = mfma32(ao, pb[m2], dvT);
        dkT = mfma32(aq, sb[m2], dkT);
      }
      cur_rt ^= 1;
      t++;
    };

    step(std::integral_constant<int, 0>{});
    // (the steps stay behind run-time branches on an opaque copy of the step count: as one
    // straight block the compiler's register allocation of the six steps spills)
    if (ns_rt > 1) step(std::integral_constant<int, 1 < NS ? 1 : 0>{});
    if (ns_rt > 2) step(std::integral_constant<int, 2 < NS ? 2 : 0>{});
    if (ns_rt > 3) step(std::integral_constant<int, 3 < NS ? 3 : 0>{});
    if (ns_rt > 4) step(std::integral_constant<int, 4 < NS ? 4 : 0>{});
    if (ns_rt > 5) step(std::integral_constant<int, 5 < NS ? 5 : 0>{});
    static_assert(NS >= 1 && NS <= kBwdMaxSteps && kBwdMaxSteps == 6, "at most six unrolled steps");
    rr_cur = rr_next;

    // end of slice i: dK^T and dV^T summed over the four query lanes as ((p0 + p1) + p2) + p3.
    // The waves put their dK^T partial into their own item buffer of the slice's last item (free
    // until the prefetch that follows the next slice's first barrier) and their dV^T partial into
    // a dedicated LDS area (whose readers of the previous slice passed this slice's first barrier
    // before any writer got here); then one barrier.  At D = 32 every wave writes and the four
    // query lanes share the sums and the stores, lane p taking channel group p (4 registers) of
    // both dK and dV; at D = 16 the p = 1..3 waves write and the p = 0 waves sum and store
    // (measured faster for each head dimension).
    // A partial is stored as NR/4 chunks of [64 lanes][4 registers]: chunk c holds registers
    // 4c..4c+3 of every lane, 16 contiguous bytes per lane (one conflict-free 16-byte access).
    const int xb = cur_rt ^ 1;  // item buffer of the slice's last item
    lf32x4* red = (lf32x4*)(lds + oRED);
    if constexpr (kShared) {
      {
        lf32x4* kx = (lf32x4*)(lds + (w * 2 + xb) * kWB) + l;
        lf32x4* vx = red + (kh * 4 + p) * (NR / 4 * 64) + l;
#pragma unroll
        for (int c = 0; c < NR / 4; c++) {
          kx[c * 64] = f32x4{dkT[4 * c], dkT[4 * c + 1], dkT[4 * c + 2], dkT[4 * c + 3]};
          vx[c * 64] = f32x4{dvT[4 * c], dvT[4 * c + 1], dvT[4 * c + 2], dvT[4 * c + 3]};
        }
      }
      lds_barrier();
      if (any_key) {
#pragma unroll
        for (int arr = 0; arr < 2; arr++) {  // 0: dK, 1: dV; channel group p (chunk p)
          f32x4 acc4;
#pragma unroll
          for (int pp = 0; pp < 4; pp++) {
            const lf32x4* src = arr == 0 ? (const lf32x4*)(lds + ((pp * 2 + kh) * 2 + xb) * kWB) + l
                                         : red + (kh * 4 + pp) * (NR / 4 * 64) + l;
            const f32x4 x = src[p * 64];
            acc4 = pp == 0 ? x : acc4 + x;
          }
          if (kok) {  // (the lane offset is recomputed here rather than kept across the slice loop)
            const int lh = lane_here();
            if (CHUNKED) {  // FP32 partials of this chunk, unscaled
              const int64_t rows = (int64_t)B * N * H * N;
              float* dst = Ck.dkvp + ((int64_t)(2 * chunk + arr) * rows + sl_row * N + kb * 64) * D;
              const unsigned lo = (unsigned)(((kh * 32 + (lh & 31)) * D + p * 8 + (lh >> 5) * 4) * 4);
              *(f32x4*)((char*)dst + lo) = acc4;
            } else {
              bf16x4 o4;
#pragma unroll
              for (int e = 0; e < 4; e++) o4[e] = (bf16)(arr == 0 ? acc4[e] * alpha : acc4[e]);
              const unsigned lo = (unsigned)(((kh * 32 + (lh & 31)) * sT + p * 8 + (lh >> 5) * 4) * 2);
              const int64_t rb = sbase + (int64_t)kb * 64 * sT;
              *(bf16x4*)((char*)((arr == 0 ? dk : dv) + rb) + lo) = o4;
            }
          }
        }
      }
    } else {
      if (p != 0) {
        lf32x4* kx = (lf32x4*)(lds + (w * 2 + xb) * kWB) + l;
        lf32x4* vx = red + (kh * 3 + p - 1) * (NR / 4 * 64) + l;
#pragma unroll
        for (int c = 0; c < NR / 4; c++) {
          kx[c * 64] = f32x4{dkT[4 * c], dkT[4 * c + 1], dkT[4 * c + 2], dkT[4 * c + 3]};
          vx[c * 64] = f32x4{dvT[4 * c], dvT[4 * c + 1], dvT[4 * c + 2], dvT[4 * c + 3]};
        }
      }
      lds_barrier();
      if (p == 0 && any_key) {
#pragma unroll
        for (int pp = 1; pp < 4; pp++) {
          const lf32x4* kx = (const lf32x4*)(lds + ((pp * 2 + kh) * 2 + xb) * kWB) + l;
          const lf32x4* vx = red + (kh * 3 + pp - 1) * (NR / 4 * 64) + l;
#pragma unroll
          for (int c = 0; c < NR / 4; c++) {
            const f32x4 k4 = kx[c * 64], v4 = vx[c * 64];
#pragma unroll
            for (int e = 0; e < 4; e++) {
              dkT[4 * c + e] += k4[e];
              dvT[4 * c + e] += v4[e];
            }
          }
        }
        if (CHUNKED) {  // FP32 partials of this chunk, unscaled
          const int64_t rows = (int64_t)B * N * H * N;
          float* pk = Ck.dkvp + ((int64_t)(2 * chunk) * rows + sl_row * N + kb * 64) * D;
          float* pv = pk + rows * D;
#pragma unroll
          for (int R = 0; R < NR / 4; R++) {
            f32x4 k4, v4;
#pragma unroll
            for (int e = 0; e < 4; e++) {
              k4[e] = dkT[R * 4 + e];
              v4[e] = dvT[R * 4 + e];
            }
            if (kok) {
              const int lh = lane_here();
              const unsigned lo = (unsigned)(((kh * 32 + (lh & 31)) * D + R * 8 + (lh >> 5) * 4) * 4);
              *(f32x4*)((char*)pk + lo) = k4;
              *(f32x4*)((char*)pv + lo) = v4;
            }
          }
        } else {
#pragma unroll
          for (int R = 0; R < NR / 4; R++) {
            bf16x4 ok4, ov4;
#pragma unroll
            for (int e = 0; e < 4; e++) {
              ok4[e] = (bf16)(dkT[R * 4 + e] * alpha);
              ov4[e] = (bf16)dvT[R * 4 + e];
            }
            if (kok) {  // (the lane offset is recomputed here rather than kept across the slice loop)
              const int lh = lane_here();
              const unsigned lo = (unsigned)(((kh * 32 + (lh & 31)) * sT + R * 8 + (lh >> 5) * 4) * 2);
              const int64_t rb = sbase + (int64_t)kb * 64 * sT;
              *(bf16x4*)((char*)(dk + rb) + lo) = ok4;
              *(bf16x4*)((char*)(dv + rb) + lo) = ov4;
            }
          }
        }
      }
    }
  }
  // write this group's pair-bias gradient partial: dbp[grp][b][h][j][k]
  float* dst = dbp + (((int64_t)grp * B + b) * H + h) * (int64_t)N * N;
#pragma unroll
  for (int s = 0; s < NS; s++) {
#pragma unroll
    for (int r = 0; r < 16; r++) {
      const int jj = (s_base + s) * 128 + p * 32 + (r >> 2) * 8 + g * 4 + (r & 3);
      if (jj < N && kok) dst[(int64_t)jj * N + kg] = face[s][r];
    }
  }
}

// ------------------------------------------------------------------ backward: dQ and D
// dq[j] = alpha * sum_k dS[j,k] K[k] for the queries of one slice (b,i,h), with P and dS
// recomputed from the forward's statistics: P = exp2(c1 S + log2e bias - lse2), dS = P (dP - D).
// This kernel runs first in the backward and also forms the correction D[j] = sum_c dO (o + r)
// of its queries, writing the row statistics the key-tile kernel streams: 16 bytes per query
// of a slice-head row, the three bf16 parts (split3_bf16) of -lse/alpha and a zero, then those
// of -D and a zero (zeros past N; -2^100 in place of -lse/alpha for a row with no finite score).
// The work-group and its key loop have the forward's shape: 4 waves = 128 queries, wave w owns
// 32 of them, and 64-key tiles of K and V stream through double-buffered LDS.  S^T = K Q^T
// (starting from the prepared bias/alpha tile) and dP^T = V dO^T run on 32x32x16 MFMA, each lane
// holding one query column and 16 keys per 32-key tile, so a query's -lse2 and -D are one
// register of its lane.  Values constant along one side of a score tile enter the accumulator
// through one k = 8 product instead of an operation per element: -D of each query column
// (the bf16 parts of split3_bf16 against ones) starts the dP^T accumulator, and a masked key's
// row of S^T gets -2^100 (its probabilities underflow to exactly zero).
// dQ^T (channels x queries) += K^T dS^T is the forward's O^T += V^T P^T
// with K in place of V and dS in place of P: the score accumulator's layout is already that of
// the product's B operand, so dS needs no trip through LDS, and the sum over all keys stays in
// an FP32 accumulator, in key order, rounded once.
template <int D, bool MASK, bool STRIDED>
__global__ __launch_bounds__(256, 4)
void dq_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
               const bf16* __restrict__ dO, const float* __restrict__ biasF, const uint8_t* __restrict__ mask,
               const bf16* __restrict__ o, const bf16* __restrict__ res, const float* __restrict__ lse,
               unsigned* __restrict__ LDp, bf16* __restrict__ dq, int B, int N, int H, float alpha, TokLayout Lg) {
  const TokLayout L = tok_layout<STRIDED, D>(Lg, N, H);
  constexpr int KT = 64;        // keys per iteration
  constexpr int NC = D / 16;    // 16-wide channel chunks
  constexpr int CPR = D / 8;    // 16-byte chunks per row
  __shared__ __attribute__((aligned(16))) bf16 Ks_[2][KT * D];
  __shared__ __attribute__((aligned(16))) bf16 Vs_[2][KT * D];
  __shared__ __attribute__((aligned(16))) uint8_t Ms_[2][KT];

  const int QT = (N + 127) / 128;
  const int64_t ntiles = (int64_t)B * H * N * QT;
  const int64_t tile = xcd_tile(ntiles);
  if (tile >= ntiles) return;
  // the forward's tile order: the work-groups on one XCD share one head's bias tiles in its L2
  const int qt = (int)(tile % QT);
  int64_t rest = tile / QT;
  const int i = (int)(rest % N); rest /= N;
  const int h = (int)(rest % H);
  const int b = (int)(rest / H);

  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, g = l >> 5, ln = l & 31;
  const int64_t sbase = L.slice(b, i, h);
  const int sT = L.sT;
  const int j = qt * 128 + w * 32 + ln;  // this lane's query
  const bool jok = j < N;
  const int Kp = (int)round_up(N, 64), Jp = (int)round_up(N, 128);
  const float* btile = biasF + ((int64_t)(b * H + h) * (Jp / 32) + (qt * 4 + w)) * (int64_t)(Kp / 32) * 1024;
  const float c1 = alpha * kLog2e;
  const uint8_t* mrow = MASK ? mask + ((int64_t)b * N + i) * N : nullptr;

  const i32x4 rk = raw_rsrc(k + sbase, L.span_bytes(N, D)), rv = raw_rsrc(v + sbase, L.span_bytes(N, D));
  const unsigned kv_vo = (unsigned)(((tid / CPR) * sT + ((tid % CPR) ^ swz<D>(tid / CPR)) * 8) * 2);
  auto prefetch = [&](int kt, int buf, float after) {
    if (w < KT * CPR / 64) {
      dma16_asm_after(rk, kv_vo, kt * KT * sT * 2, lds_addr(&Ks_[buf][w * 512]), after);
      dma16_asm_after(rv, kv_vo, kt * KT * sT * 2, lds_addr(&Vs_[buf][w * 512]), after);
    }
  };

  // this lane's query row of Q and dO (B operands of the two score products); the lane pair
  // (l, l^32) holds the row's channels cc*16 + 0..7 and cc*16 + 8..15
  bf16x8 qf[NC], df[NC];
#pragma unroll
  for (int cc = 0; cc < NC; cc++) {
    qf[cc] = jok ? *(const bf16x8*)(q + sbase + (int64_t)j * sT + cc * 16 + g * 8) : zero8();
    df[cc] = jok ? *(const bf16x8*)(dO + sbase + (int64_t)j * sT + cc * 16 + g * 8) : zero8();
  }
  // The correction D[j] = sum_c dO * (o + residual) in FP32 (dO * o without a residual): the
  // lane's channels in ascending pairs, each pair's dO.o then dO.r products (exact in FP32)
  // summed by one two-term dot instruction, then the lane pair's two sums.  -lse2 = -lse * log2(e).
  // The row statistics for the key-tile kernel, which runs after this one, hold the bf16 parts
  // of -lse/alpha and of -D (zero past N).
  float dsum = 0.0f;
  if (jok) {
#pragma unroll
    for (int cc = 0; cc < NC; cc++) {
      const int64_t off = sbase + (int64_t)j * sT + cc * 16 + g * 8;
      const bf16x8 ov = ld_nt((const bf16x8*)(o + off));
      if (res) {
        const bf16x8 rv = ld_nt((const bf16x8*)(res + off));
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          dsum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{df[cc][e], df[cc][e + 1]}, bf16x2{ov[e], ov[e + 1]}, dsum, false);
          dsum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{df[cc][e], df[cc][e + 1]}, bf16x2{rv[e], rv[e + 1]}, dsum, false);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; e += 2)
          dsum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{df[cc][e], df[cc][e + 1]}, bf16x2{ov[e], ov[e + 1]}, dsum, false);
      }
    }
  }
  const float Dj = dsum + __shfl_xor(dsum, 32);  // (the same bits on both lanes of the pair)
  const int64_t srow = ((int64_t)b * N + i) * H + h;  // slice-head row
  const float lse_j = jok ? lse[srow * N + j] : 0.0f;
  const float inv_alpha = 1.0f / alpha;
  const float nl2 = -lse_j * kLog2e;
  const u32x2v dsp = split3_bf16(-Dj);
  if (g == 0) {
    const u32x2v lsp = split3_bf16(lse_j == INFINITY ? -0x1p100f : -lse_j * inv_alpha);
    *(u32x4v*)(LDp + (srow * Jp + j) * 4) = u32x4v{lsp.x, lsp.y, dsp.x, dsp.y};
  }
  // B operand of the -D start product (parts at k = 0..2 of this lane's query column; the upper
  // lane half holds k = 4..7, zero) and its A operand (ones at k = 0..2 in every key row)
  const u32x2v dB = g == 0 ? dsp : u32x2v{0u, 0u};
  // at D = 16 (one product per dP^T tile) the registers allow -D itself as the product's start
  // value: every accumulator register of a lane belongs to its query column
  f32x16 dstart;
  if constexpr (D == 16) {
#pragma unroll
    for (int r = 0; r < 16; r++) dstart[r] = -Dj;
  }

  f32x16 acc = {};
  const int nkt = (N + KT - 1) / KT;
  const int G16 = l >> 4, chalf = G16 & 1;
  // A operand of the -D start product: ones at k = 0..2 in every key row (lanes of the upper k
  // half hold k = 4..7, zero)
  const u32x2v one3 = g == 0 ? u32x2v{0x3F803F80u, 0x3F80u} : u32x2v{0u, 0u};
  // Key tile kt in LDS buffer CUR.  The buffer index is a compile-time constant (the loop below
  // runs two tiles per pass), so every LDS address is a per-lane offset plus an immediate.
  auto key_tile = [&](int kt, auto cur_) {
    constexpr int cur = decltype(cur_)::value;
    // the next tile's key-mask bytes, loaded ahead of the bias loads (and so covered by the wait
    // below) and stored right after the barrier, to be read after the next one
    uint8_t mnext = 1;
    if (MASK && kt + 1 < nkt && tid < KT && (kt + 1) * KT + tid < N) mnext = mrow[(kt + 1) * KT + tid];
    // this wave's bias tiles of tile kt: eight 16-byte loads into the score accumulators
    f32x16 s[2];
#pragma unroll
    for (int tt = 0; tt < 2; tt++) {
#pragma unroll
      for (int R = 0; R < 4; R++) {
        const f32x4 bv = *(const f32x4*)(btile + (int64_t)(kt * 2 + tt) * 1024 + ((R * 2 + g) * 32 + ln) * 4);
        s[tt][R * 4 + 0] = bv[0]; s[tt][R * 4 + 1] = bv[1];
        s[tt][R * 4 + 2] = bv[2]; s[tt][R * 4 + 3] = bv[3];
      }
    }
    // every load but those eight, among them this wave's part of tile kt, has landed
    asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    __syncthreads();  // all of tile kt is in LDS; buffer cur^1 is free
    if (MASK && tid < KT) Ms_[cur ^ 1][tid] = mnext;
    // the next tile's K and V, issued once the bias loads have landed (an operand of the
    // statement is one of their values), so that the compiler's waits for them never include it
    if (kt + 1 < nkt) prefetch(kt + 1, cur ^ 1, s[1][15]);
    const lbf16* Ks = (const lbf16*)Ks_[cur];
    const lbf16* Vs = (const lbf16*)Vs_[cur];

#pragma unroll
    for (int tt = 0; tt < 2; tt++) {
      const int rk_ = tt * 32 + ln;
      f32x16 dp;
#pragma unroll
      for (int cc = 0; cc < NC; cc++) {
        const bf16x8 ka = *(const lbf16x8*)(Ks + rk_ * D + ((cc * 2 + g) ^ swz<D>(rk_)) * 8);
        const bf16x8 va = *(const lbf16x8*)(Vs + rk_ * D + ((cc * 2 + g) ^ swz<D>(rk_)) * 8);
        s[tt] = mfma32(ka, qf[cc], s[tt]);
        if constexpr (D == 16) {
          dp = mfma32(va, df[cc], dstart);  // dP - D
        } else {
          dp = mfma32(va, df[cc], cc == 0 ? f32x16{} : dp);
          if (cc == 0) dp = mfma32k8(one3, dB, dp);  // dP - D
        }
      }
      if (MASK) {  // A: -2^100 at k = 0 of a masked key's row (this lane's row is key rk_); B: one at k = 0
        const u32x2v mA = {(g == 0 && !Ms_[cur][rk_]) ? 0xF180u : 0u, 0u};
        s[tt] = mfma32k8(mA, u32x2v{one3.x & 0xFFFFu, 0u}, s[tt]);
      }
      float ds[16];
#pragma unroll
      for (int r = 0; r < 16; r++) ds[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[tt][r], c1, nl2)) * dp[r];
      // dQ^T += K^T dS^T; lane group (l/16) selects channel half and key run (at D = 16 both
      // halves read channels 0..15: the upper 16 rows of the product repeat the lower ones and
      // are never stored)
#pragma unroll
      for (int m2 = 0; m2 < 2; m2++) {
        const bf16x8 sb = pack8(&ds[m2 * 8]);
        const int r0 = tt * 32 + m2 * 16 + g * 4;
        const int c0 = D == 32 ? chalf * 16 : 0;
        const bf16x8 a = cat8(tr16p(Ks + tr_off<D>(l, r0, c0)), tr16p(Ks + tr_off<D>(l, r0 + 8, c0)));
        acc = mfma32(a, sb, acc);
      }
    }
  };
  if (MASK && tid < KT) Ms_[0][tid] = tid < N ? mrow[tid] : (uint8_t)1;
  prefetch(0, 0, 0.0f);
  for (int kt = 0; kt < nkt; kt += 2) {
    key_tile(kt, std::integral_constant<int, 0>{});
    if (kt + 1 < nkt) key_tile(kt + 1, std::integral_constant<int, 1>{});
  }

  if (jok) {
    bf16* drow = dq + sbase + (int64_t)j * sT;
#pragma unroll
    for (int R = 0; R < D / 8; R++) {
      bf16x4 ob;
#pragma unroll
      for (int e = 0; e < 4; e++) ob[e] = (bf16)(acc[R * 4 + e] * alpha);
      *(bf16x4*)(drow + R * 8 + g * 4) = ob;
    }
  }
}

// Chunked backward: dk = bf16(alpha * sum_c partial[c]), dv = bf16(sum_c partial[c]), chunks in
// ascending order, in FP32.  One thread per 4 channels of one key row of one slice-head.
template <int D, bool STRIDED>
__global__ __launch_bounds__(256)
void reduce_dkv_kernel(const float* __restrict__ dkvp, bf16* __restrict__ dk, bf16* __restrict__ dv, int N, int H,
                       int nqc, int64_t rows, float alpha, TokLayout Lg) {
  const TokLayout L = tok_layout<STRIDED, D>(Lg, N, H);
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= rows * (D / 4)) return;
  const int64_t row = t / (D / 4);  // (slice-head row) * N + key
  const int c = (int)(t % (D / 4)) * 4;
  f32x4 sk = {}, sv = {};
  for (int ch = 0; ch < nqc; ch++) {
    const f32x4 a = __builtin_nontemporal_load((const f32x4*)(dkvp + ((int64_t)(2 * ch) * rows + row) * D + c));
    const f32x4 b = __builtin_nontemporal_load((const f32x4*)(dkvp + ((int64_t)(2 * ch + 1) * rows + row) * D + c));
    sk += a;
    sv += b;
  }
  const int64_t sl = row / N;
  const int key = (int)(row % N);
  const int64_t bi = sl / H;
  const int64_t off = L.slice((int)(bi / N), (int)(bi % N), (int)(sl % H)) + (int64_t)key * L.sT + c;
  bf16x4 ok, ov;
#pragma unroll
  for (int e = 0; e < 4; e++) {
    ok[e] = (bf16)(sk[e] * alpha);
    ov[e] = (bf16)sv[e];
  }
  *(bf16x4*)(dk + off) = ok;
  *(bf16x4*)(dv + off) = ov;
}

// VEC: four adjacent elements per thread (n divisible by 4, so every partial stays 16-byte aligned)
template <bool VEC>
__global__ __launch_bounds__(256)
void reduce_dbias_kernel(const float* __restrict__ dbp, float* __restrict__ dbias, int ngroups, int64_t n) {
  typedef typename std::conditional<VEC, f32x4, float>::type T;
  constexpr int W = VEC ? 4 : 1, U = 8;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t * W >= n) return;
  T s = {};
  for (int g0 = 0; g0 < ngroups; g0 += U) {
    T x[U];
#pragma unroll
    for (int u = 0; u < U; u++) x[u] = __builtin_nontemporal_load((const T*)(dbp + (int64_t)min(g0 + u, ngroups - 1) * n + t * W));
#pragma unroll
    for (int u = 0; u < U; u++) {
      if (g0 + u == 0) s = x[u];
      else if (g0 + u < ngroups) s += x[u];
    }
  }
  *(T*)(dbias + t * W) = s;
}

// ------------------------------------------------------------------ host side

struct Plan {
  int64_t B, N, H, D;
  int64_t Kp, Jp;           // padded key / query extents of the prepared bias
  int64_t KB;               // 64-key blocks
  int64_t ngroups, G;       // slice groups of the backward and slices per group
  int64_t elems;            // B*N*H*N*D
  int64_t rows;             // B*N*H*N
  int64_t bias_f32_bytes;   // prepared forward bias (FP32 tiles)
  int64_t bias_b16_bytes;   // prepared backward bias (bf16 column blocks)
  int64_t nst, nqc;          // 128-query steps per slice; query chunks of the backward
  int64_t cs, n1;            // steps of the longest chunks, and how many chunks have cs steps
  int64_t off_LD, off_bF, off_dbp, off_dkv, bwd_bytes;
};

constexpr int64_t kAlign = 256;

// (the last bound keeps every grid and the 16-query tile index of the dq reduction in 32 bits)
// max_n: TRI_ATTN_FWD_MAX_N for the forward, TRI_ATTN_MAX_N for the backward (whose work-group
// keeps the pair-bias gradient of all N queries of its key block in registers)
bool shape_ok(int64_t B, int64_t N, int64_t H, int64_t D, int64_t max_n) {
  return B >= 1 && N >= 1 && H >= 1 && (D == 16 || D == 32) && N <= max_n && B <= (1 << 20) &&
         H <= (1 << 12) && B * N * H * (round_up(N, 128) / 16) <= INT32_MAX;
}

Plan make_plan(int64_t B, int64_t N, int64_t H, int64_t D) {
  Plan p{};
  p.B = B; p.N = N; p.H = H; p.D = D;
  p.Kp = round_up(N, 64);
  p.Jp = round_up(N, 128);
  p.KB = (N + 63) / 64;
  p.nst = p.Jp / 128;
  p.nqc = (p.nst + kBwdMaxSteps - 1) / kBwdMaxSteps;
  p.cs = (p.nst + p.nqc - 1) / p.nqc;
  p.n1 = p.nst - (p.cs - 1) * p.nqc;
  {
    // Slice groups of the backward: each work-group runs a whole slice group, one per CU, so a
    // launch takes ceil(work-groups / CUs) rounds of (slices per group) x (chunk steps).  Pick
    // the group count that minimises that time (about 1.6 us per slice and 128-query step)
    // plus the round trip of one FP32 pair-bias partial per group (B*H*N*N*4 bytes written
    // and read at about 5.5 TB/s).
    constexpr int64_t kCUs = 256;
    double best = 0.0;
    int64_t bestG = N;
    for (int64_t g = 1; g <= std::min<int64_t>(N, 256); g++) {
      const int64_t G = (N + g - 1) / g, ng = (N + G - 1) / G;
      if (ng != g) continue;  // same partition as a smaller g
      const int64_t tiles = B * H * p.KB * ng;
      int64_t units = ((p.n1 * tiles + kCUs - 1) / kCUs) * p.cs * G;
      if (p.n1 < p.nqc) units += (((p.nqc - p.n1) * tiles + kCUs - 1) / kCUs) * (p.cs - 1) * G;
      const double t = (double)units * 1.6e-6 + (double)ng * (double)(B * H * N * N) * 8.0 / 5.5e12;
      if (g == 1 || t < best) {
        best = t;
        bestG = G;
      }
    }
    p.G = bestG;
  }
  p.ngroups = (N + p.G - 1) / p.G;
  p.elems = B * N * H * N * D;
  p.rows = B * N * H * N;
  p.bias_f32_bytes = round_up(B * H * p.Kp * p.Jp * 4, kAlign);
  p.bias_b16_bytes = round_up(B * H * p.Kp * p.Jp * 2, kAlign);
  // backward workspace: fp16 bias column blocks | row statistics | FP32 bias/alpha tiles (the dQ
  // kernel's, as the forward's) | pair-bias gradient partials | chunked dK / dV partials
  p.off_LD = p.bias_b16_bytes;
  p.off_bF = p.off_LD + round_up(B * N * H * p.Jp * 16, kAlign);
  p.off_dbp = p.off_bF + p.bias_f32_bytes;
  p.off_dkv = p.off_dbp + round_up(p.ngroups * B * H * N * N * 4, kAlign);
  // FP32 dK / dV partials per query chunk, only when there is more than one chunk
  p.bwd_bytes = p.off_dkv + (p.nqc > 1 ? round_up(2 * p.nqc * p.elems * 4, kAlign) : 0);
  return p;
}

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

// Strides of the token tensors for each layout.  Only the addressing differs: every kernel
// runs the same work in the same order, so a layout changes no result bit.
bool make_layout(int layout, const Plan& P, TokLayout* L) {
  const int64_t N = P.N, H = P.H, D = P.D;
  switch (layout) {
    case TRI_ATTN_LAYOUT_SLICE_HEAD: *L = {N * H * N * D, H * N * D, N * D, (int)D}; break;
    case TRI_ATTN_LAYOUT_PAIR_START: *L = {N * N * H * D, N * H * D, D, (int)(H * D)}; break;
    case TRI_ATTN_LAYOUT_PAIR_END: *L = {N * N * H * D, H * D, D, (int)(N * H * D)}; break;
    default: return false;
  }
  return true;
}

// The buffer descriptors address a slice-head's rows with 32-bit offsets, including the
// padded rows up to the next multiple of 128 (those read as zeros).
bool layout_fits(const TokLayout& L, const Plan& P) { return (P.Jp * L.sT + P.D) * 2 <= INT32_MAX; }

struct Range { const void* p; int64_t n; bool out; };

bool overlaps(const Range* r, int n) {
  for (int a = 0; a < n; a++) {
    if (!r[a].p || r[a].n <= 0) continue;
    for (int c = a + 1; c < n; c++) {
      if (!r[c].p || r[c].n <= 0) continue;
      if (!r[a].out && !r[c].out) continue;  // inputs may alias each other
      const uintptr_t a0 = (uintptr_t)r[a].p, a1 = a0 + (uintptr_t)r[a].n;
      const uintptr_t c0 = (uintptr_t)r[c].p, c1 = c0 + (uintptr_t)r[c].n;
      if (a0 < c1 && c0 < a1) return true;
    }
  }
  return false;
}

unsigned grid_xcd(int64_t ntiles) { return (unsigned)(round_up(ntiles, kXcd)); }

template <int D, bool STRIDED>
tri_attn_status launch_fwd(unsigned stages, const Plan& P, const TokLayout& L, const void* q, const void* k,
                           const void* v, const void* bias, const uint8_t* mask, void* o, float* lse, void* res,
                           void* ws, hipStream_t st) {
  const float alpha = 1.0f / sqrtf((float)D);
  float* biasF = (float*)ws;
  const int64_t nb = P.B * P.H * P.Jp * P.Kp;
  if (stages & TRI_ATTN_STAGE_PREP)
    hipLaunchKernelGGL(bias_prep_fwd_kernel, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0, st,
                       (const bf16*)bias, biasF, (int)P.N, (int)P.Jp, (int)P.Kp, 1.0f / alpha, nb);
  const int64_t ntiles = P.B * P.H * P.N * ((P.N + 127) / 128);
  if (!(stages & TRI_ATTN_STAGE_MAIN)) {
  } else if (mask)
    hipLaunchKernelGGL((fwd_kernel<D, true, STRIDED>), dim3(grid_xcd(ntiles)), dim3(256), 0, st, (const bf16*)q,
                       (const bf16*)k, (const bf16*)v, biasF, mask, (bf16*)o, lse, (bf16*)res, (int)P.B, (int)P.N,
                       (int)P.H, alpha, L);
  else
    hipLaunchKernelGGL((fwd_kernel<D, false, STRIDED>), dim3(grid_xcd(ntiles)), dim3(256), 0, st, (const bf16*)q,
                       (const bf16*)k, (const bf16*)v, biasF, mask, (bf16*)o, lse, (bf16*)res, (int)P.B, (int)P.N,
                       (int)P.H, alpha, L);
  return hipGetLastError() == hipSuccess ? TRI_ATTN_SUCCESS : TRI_ATTN_ERROR_LAUNCH;
}

template <int D, bool STRIDED>
tri_attn_status launch_bwd(unsigned stages, const Plan& P, const TokLayout& L, const void* q, const void* k,
                           const void* v, const void* bias, const uint8_t* mask, const void* o, const float* lse,
                           const void* res, const void* dO, void* dq, void* dk, void* dv, float* dbias, void* ws,
                           hipStream_t st) {
  const float alpha = 1.0f / sqrtf((float)D);
  char* base = (char*)ws;
  bf16* biasB = (bf16*)base;
  unsigned* LDg = (unsigned*)(base + P.off_LD);
  float* biasF = (float*)(base + P.off_bF);
  float* dbp = (float*)(base + P.off_dbp);
  const int64_t nb = P.B * P.H * P.Kp * P.Jp;
  if (stages & TRI_ATTN_STAGE_PREP) {
    hipLaunchKernelGGL(bias_prep_bwd_kernel, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0, st,
                       (const bf16*)bias, (_Float16*)biasB, biasF, (int)P.N, (int)P.Jp, (int)P.Kp, (int)P.KB,
                       (int)(P.Jp / 128), 1.0f / alpha, nb);
    // dq, and the correction D with the row statistics the key-tile kernel reads
    const int64_t qtiles = P.B * P.H * P.N * ((P.N + 127) / 128);
    if (mask)
      hipLaunchKernelGGL((dq_kernel<D, true, STRIDED>), dim3(grid_xcd(qtiles)), dim3(256), 0, st, (const bf16*)q,
                         (const bf16*)k, (const bf16*)v, (const bf16*)dO, biasF, mask, (const bf16*)o,
                         (const bf16*)res, lse, LDg, (bf16*)dq, (int)P.B, (int)P.N, (int)P.H, alpha, L);
    else
      hipLaunchKernelGGL((dq_kernel<D, false, STRIDED>), dim3(grid_xcd(qtiles)), dim3(256), 0, st, (const bf16*)q,
                         (const bf16*)k, (const bf16*)v, (const bf16*)dO, biasF, mask, (const bf16*)o,
                         (const bf16*)res, lse, LDg, (bf16*)dq, (int)P.B, (int)P.N, (int)P.H, alpha, L);
  }
  float* dkvp = (float*)(base + P.off_dkv);
  if (stages & TRI_ATTN_STAGE_MAIN) {
    const int64_t per_chunk = P.B * P.H * P.ngroups * P.KB;
    auto launch = [&](auto ns_, auto chunked_, int c_begin, int ncl, int step0) {
      constexpr int NS = decltype(ns_)::value;
      constexpr bool CH = decltype(chunked_)::value;
      const Chunking ck{(int)P.nst, c_begin, ncl, step0, dkvp};
      const dim3 grid(grid_xcd(per_chunk * ncl));
      if (mask)
        hipLaunchKernelGGL((bwd_kernel<D, true, NS, STRIDED, CH>), grid, dim3(512), 0, st, (const bf16*)q,
                           (const bf16*)k, (const bf16*)v, (const bf16*)dO, biasB, mask, LDg, dbp, (bf16*)dk,
                           (bf16*)dv, (int)P.B, (int)P.N, (int)P.H, (int)P.G, (int)P.ngroups, alpha, L, ck);
      else
        hipLaunchKernelGGL((bwd_kernel<D, false, NS, STRIDED, CH>), grid, dim3(512), 0, st, (const bf16*)q,
                           (const bf16*)k, (const bf16*)v, (const bf16*)dO, biasB, mask, LDg, dbp, (bf16*)dk,
                           (bf16*)dv, (int)P.B, (int)P.N, (int)P.H, (int)P.G, (int)P.ngroups, alpha, L, ck);
    };
    auto by_steps = [&](int ns, auto chunked_, int c_begin, int ncl, int step0) {
      switch (ns) {  // 128-query steps of the chunk (1..6)
        case 1: launch(std::integral_constant<int, 1>{}, chunked_, c_begin, ncl, step0); break;
        case 2: launch(std::integral_constant<int, 2>{}, chunked_, c_begin, ncl, step0); break;
        case 3: launch(std::integral_constant<int, 3>{}, chunked_, c_begin, ncl, step0); break;
        case 4: launch(std::integral_constant<int, 4>{}, chunked_, c_begin, ncl, step0); break;
        case 5: launch(std::integral_constant<int, 5>{}, chunked_, c_begin, ncl, step0); break;
        default: launch(std::integral_constant<int, 6>{}, chunked_, c_begin, ncl, step0); break;
      }
    };
    if (P.nqc == 1) {
      by_steps((int)P.nst, std::false_type{}, 0, 1, 0);
    } else {  // chunks as equal as possible: n1 chunks of cs steps, then chunks of cs - 1
      const int nqc = (int)P.nqc, cs = (int)P.cs, n1 = (int)P.n1;
      by_steps(cs, std::true_type{}, 0, n1, 0);
      if (n1 < nqc) by_steps(cs - 1, std::true_type{}, n1, nqc - n1, n1 * cs);
    }
  }
  if (stages & TRI_ATTN_STAGE_FINAL) {
    const int64_t nbias = P.B * P.H * P.N * P.N;
    if (nbias % 4 == 0)
      hipLaunchKernelGGL(reduce_dbias_kernel<true>, dim3((unsigned)((nbias / 4 + 255) / 256)), dim3(256), 0, st, dbp,
                         dbias, (int)P.ngroups, nbias);
    else
      hipLaunchKernelGGL(reduce_dbias_kernel<false>, dim3((unsigned)((nbias + 255) / 256)), dim3(256), 0, st, dbp,
                         dbias, (int)P.ngroups, nbias);
    if (P.nqc > 1) {
      const int64_t nt = P.rows * (D / 4);
      hipLaunchKernelGGL((reduce_dkv_kernel<D, STRIDED>), dim3((unsigned)((nt + 255) / 256)), dim3(256), 0, st, dkvp,
                         (bf16*)dk, (bf16*)dv, (int)P.N, (int)P.H, (int)P.nqc, P.rows, alpha, L);
    }
  }
  return hipGetLastError() == hipSuccess ? TRI_ATTN_SUCCESS : TRI_ATTN_ERROR_LAUNCH;
}

// ------------------------------------------------------------------ allocation-free forward
// Device-resident scratch of tri_attn_fwd_noalloc: the prepared forward bias tiles of one call.
// The runtime gives every GPU the library runs on its own copy, at its own address, held until
// the process ends.  In host code `scratch` names a host-side stand-in, never a device address:
// the address a kernel may use comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[TRI_ATTN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch (looked up on the first call per device).
tri_attn_status current_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return TRI_ATTN_ERROR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return TRI_ATTN_ERROR_LAUNCH;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return TRI_ATTN_SUCCESS;
}

}  // namespace

extern "C" {

const char* tri_attn_status_string(int status) {
  switch (status) {
    case TRI_ATTN_ERROR_SCRATCH_LIMIT: return "TRI_ATTN_ERROR_SCRATCH_LIMIT";
    case TRI_ATTN_SUCCESS: return "TRI_ATTN_SUCCESS";
    case TRI_ATTN_ERROR_INVALID_VALUE: return "TRI_ATTN_ERROR_INVALID_VALUE";
    case TRI_ATTN_ERROR_UNSUPPORTED: return "TRI_ATTN_ERROR_UNSUPPORTED";
    case TRI_ATTN_ERROR_MISALIGNED: return "TRI_ATTN_ERROR_MISALIGNED";
    case TRI_ATTN_ERROR_WORKSPACE: return "TRI_ATTN_ERROR_WORKSPACE";
    case TRI_ATTN_ERROR_LAUNCH: return "TRI_ATTN_ERROR_LAUNCH";
    default: return "TRI_ATTN_UNKNOWN_STATUS";
  }
}

size_t tri_attn_fwd_workspace_bytes(int64_t B, int64_t N, int64_t H, int64_t D) {
  if (!shape_ok(B, N, H, D, TRI_ATTN_FWD_MAX_N)) return 0;
  return (size_t)make_plan(B, N, H, D).bias_f32_bytes;
}

size_t tri_attn_bwd_workspace_bytes(int64_t B, int64_t N, int64_t H, int64_t D) {
  if (!shape_ok(B, N, H, D, TRI_ATTN_MAX_N)) return 0;
  return (size_t)make_plan(B, N, H, D).bwd_bytes;
}

tri_attn_status tri_attn_fwd_ex(unsigned stages, int layout, int64_t B, int64_t N, int64_t H, int64_t D,
                                const void* q, const void* k, const void* v, const void* bias,
                                const uint8_t* key_mask, void* o, float* lse, void* residual, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  if (stages & ~TRI_ATTN_STAGE_ALL) return TRI_ATTN_ERROR_INVALID_VALUE;
  if (B < 1 || N < 1 || H < 1) return TRI_ATTN_ERROR_INVALID_VALUE;
  if (!shape_ok(B, N, H, D, TRI_ATTN_FWD_MAX_N)) return TRI_ATTN_ERROR_UNSUPPORTED;
  if (!q || !k || !v || !bias || !o || !lse) return TRI_ATTN_ERROR_INVALID_VALUE;
  const Plan P = make_plan(B, N, H, D);
  TokLayout L;
  if (!make_layout(layout, P, &L)) return TRI_ATTN_ERROR_INVALID_VALUE;
  if (!layout_fits(L, P)) return TRI_ATTN_ERROR_UNSUPPORTED;
  const int64_t tb = P.elems * 2, bb = B * H * N * N * 2, lb = P.rows * 4, mb = B * N * N;
  const Range rs[] = {{q, tb, false}, {k, tb, false}, {v, tb, false}, {bias, bb, false}, {key_mask, mb, false},
                      {o, tb, true}, {lse, lb, true}, {residual, tb, true}, {workspace, (int64_t)workspace_bytes, true}};
  if (overlaps(rs, 9)) return TRI_ATTN_ERROR_INVALID_VALUE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(bias) || !aligned16(o) || !aligned16(lse) ||
      (residual && !aligned16(residual)) || (workspace && !aligned16(workspace)))
    return TRI_ATTN_ERROR_MISALIGNED;
  if (!workspace || workspace_bytes < (size_t)P.bias_f32_bytes) return TRI_ATTN_ERROR_WORKSPACE;
  auto go = [&](auto d_, auto strided_) {
    return launch_fwd<decltype(d_)::value, decltype(strided_)::value>(stages, P, L, q, k, v, bias, key_mask, o, lse,
                                                                        residual, workspace, stream);
  };
  const bool strided = layout != TRI_ATTN_LAYOUT_SLICE_HEAD;
  if (D == 16) return strided ? go(std::integral_constant<int, 16>{}, std::true_type{})
                              : go(std::integral_constant<int, 16>{}, std::false_type{});
  return strided ? go(std::integral_constant<int, 32>{}, std::true_type{})
                 : go(std::integral_constant<int, 32>{}, std::false_type{});
}

tri_attn_status tri_attn_fwd_stages(unsigned stages, int64_t B, int64_t N, int64_t H, int64_t D, const void* q,
                                    const void* k, const void* v, const void* bias, const uint8_t* key_mask, void* o,
                                    float* lse, void* residual, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream) {
  return tri_attn_fwd_ex(stages, TRI_ATTN_LAYOUT_SLICE_HEAD, B, N, H, D, q, k, v, bias, key_mask, o, lse, residual,
                         workspace, workspace_bytes, stream);
}

tri_attn_status tri_attn_fwd(int64_t B, int64_t N, int64_t H, int64_t D, const void* q, const void* k, const void* v,
                             const void* bias, const uint8_t* key_mask, void* o, float* lse, void* residual,
                             void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return tri_attn_fwd_stages(TRI_ATTN_STAGE_ALL, B, N, H, D, q, k, v, bias, key_mask, o, lse, residual, workspace,
                             workspace_bytes, stream);
}

size_t tri_attn_noalloc_scratch_bytes(void) { return (size_t)TRI_ATTN_NOALLOC_SCRATCH_BYTES; }

tri_attn_status tri_attn_fwd_noalloc(int64_t B, int64_t N, int64_t H, int64_t D, const void* q, const void* k,
                                     const void* v, const void* bias, const uint8_t* key_mask, void* o, float* lse,
                                     void* residual, hipStream_t stream) {
  // host-only checks first, in the order of tri_attn_fwd_ex, then the scratch limit; no HIP call
  // is made unless all of them pass
  if (B < 1 || N < 1 || H < 1) return TRI_ATTN_ERROR_INVALID_VALUE;
  if (!shape_ok(B, N, H, D, TRI_ATTN_FWD_MAX_N)) return TRI_ATTN_ERROR_UNSUPPORTED;
  if (!q || !k || !v || !bias || !o || !lse) return TRI_ATTN_ERROR_INVALID_VALUE;
  const Plan P = make_plan(B, N, H, D);
  if (P.bias_f32_bytes > (int64_t)TRI_ATTN_NOALLOC_SCRATCH_BYTES) return TRI_ATTN_ERROR_SCRATCH_LIMIT;
  void* ws = nullptr;
  const tri_attn_status st = current_scratch(&ws);
  if (st != TRI_ATTN_SUCCESS) return st;
  return tri_attn_fwd_ex(TRI_ATTN_STAGE_ALL, TRI_ATTN_LAYOUT_SLICE_HEAD, B, N, H, D, q, k, v, bias, key_mask, o, lse,
                         residual, ws, (size_t)TRI_ATTN_NOALLOC_SCRATCH_BYTES, stream);
}

tri_attn_status tri_attn_bwd_ex(unsigned stages, int layout, int64_t B, int64_t N, int64_t H, int64_t D,
                                const void* q, const void* k, const void* v, const void* bias,
                                const uint8_t* key_mask, const void* o, const float* lse, const void* residual,
                                const void* dO, void* dq, void* dk, void* dv, float* dbias, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  if (stages & ~TRI_ATTN_STAGE_ALL) return TRI_ATTN_ERROR_INVALID_VALUE;
  if (B < 1 || N < 1 || H < 1) return TRI_ATTN_ERROR_INVALID_VALUE;
  if (!shape_ok(B, N, H, D, TRI_ATTN_MAX_N)) return TRI_ATTN_ERROR_UNSUPPORTED;
  if (!q || !k || !v || !bias || !o || !lse || !dO || !dq || !dk || !dv || !dbias) return TRI_ATTN_ERROR_INVALID_VALUE;
  const Plan P = make_plan(B, N, H, D);
  TokLayout L;
  if (!make_layout(layout, P, &L)) return TRI_ATTN_ERROR_INVALID_VALUE;
  if (!layout_fits(L, P)) return TRI_ATTN_ERROR_UNSUPPORTED;
  const int64_t tb = P.elems * 2, bb = B * H * N * N * 2, lb = P.rows * 4, mb = B * N * N, db = B * H * N * N * 4;
  const Range rs[] = {{q, tb, false},  {k, tb, false},  {v, tb, false},   {bias, bb, false},
                      {key_mask, mb, false}, {o, tb, false}, {lse, lb, false}, {residual, tb, false},
                      {dO, tb, false}, {dq, tb, true},   {dk, tb, true},    {dv, tb, true},
                      {dbias, db, true}, {workspace, (int64_t)workspace_bytes, true}};
  if (overlaps(rs, 14)) return TRI_ATTN_ERROR_INVALID_VALUE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(bias) || !aligned16(o) || !aligned16(lse) ||
      (residual && !aligned16(residual)) || !aligned16(dO) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) ||
      !aligned16(dbias) || (workspace && !aligned16(workspace)))
    return TRI_ATTN_ERROR_MISALIGNED;
  if (!workspace || workspace_bytes < (size_t)P.bwd_bytes) return TRI_ATTN_ERROR_WORKSPACE;
  auto go = [&](auto d_, auto strided_) {
    return launch_bwd<decltype(d_)::value, decltype(strided_)::value>(stages, P, L, q, k, v, bias, key_mask, o, lse,
                                                                        residual, dO, dq, dk, dv, dbias, workspace,
                                                                        stream);
  };
  const bool strided = layout != TRI_ATTN_LAYOUT_SLICE_HEAD;
  if (D == 16) return strided ? go(std::integral_constant<int, 16>{}, std::true_type{})
                              : go(std::integral_constant<int, 16>{}, std::false_type{});
  return strided ? go(std::integral_constant<int, 32>{}, std::true_type{})
                 : go(std::integral_constant<int, 32>{}, std::false_type{});
}

tri_attn_status tri_attn_bwd_stages(unsigned stages, int64_t B, int64_t N, int64_t H, int64_t D, const void* q,
                                    const void* k, const void* v, const void* bias, const uint8_t* key_mask,
                                    const void* o, const float* lse, const void* residual, const void* dO, void* dq,
                                    void* dk, void* dv, float* dbias, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream) {
  return tri_attn_bwd_ex(stages, TRI_ATTN_LAYOUT_SLICE_HEAD, B, N, H, D, q, k, v, bias, key_mask, o, lse, residual,
                         dO, dq, dk, dv, dbias, workspace, workspace_bytes, stream);
}

tri_attn_status tri_attn_bwd(int64_t B, int64_t N, int64_t H, int64_t D, const void* q, const void* k, const void* v,
                             const void* bias, const uint8_t* key_mask, const void* o, const float* lse,
                             const void* residual, const void* dO, void* dq, void* dk, void* dv, float* dbias,
                             void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return tri_attn_bwd_stages(TRI_ATTN_STAGE_ALL, B, N, H, D, q, k, v, bias, key_mask, o, lse, residual, dO, dq, dk,
                             dv, dbias, workspace, workspace_bytes, stream);
}

}  // extern "C"
