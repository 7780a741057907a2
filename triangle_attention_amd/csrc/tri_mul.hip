// tri_mul.hip — the triangle multiplication core on gfx950 (MI355X), part of libtriattn.so.
//
// Triangle multiplicative update (kongchang.com article on fast_trimul, section
// "什么是三角乘法更新"): each pair (i, j) gathers information through a third index k by an
// outer product and a reduction over k, along the rows (outgoing) or the columns (incoming)
// of the pair representation.  The cubic core computed here, for pair tensors [B, N, N, C]
// with channels last:
//   outgoing  x[i,j,c] = sum_k a[i,k,c] b[j,k,c]      incoming  x[i,j,c] = sum_k a[k,i,c] b[k,j,c]
// and the gradients of both.  All six products are one operation with different strides:
//   OUT[r, s, c] = sum_t P[r, t, c] * Q[s, t, c]
// where P and Q address their row index r (s) and reduction index t with strides that are
// either C (the second pair index) or N*C (the first), and OUT[r, s, c] sits at r*N*C + s*C + c.
//
// Kernel design.  Each channel is an independent N x N x N product, so a work-group takes a
// 64 x 64 output tile of 8 adjacent channels (one 16-byte chunk per pair entry) and each of its
// 8 waves owns one channel: four 32x32 accumulator tiles on v_mfma_f32_32x32x16_bf16.  The
// reduction runs in steps of 32.  Every thread loads 4 chunks (4 consecutive t of one row, 8
// channels each) of P and of Q for the next step while the current step's products run, then
// transposes them in registers into per-channel rows of 4 t (8 bytes) and writes them to the
// other half of a double-buffered LDS stage, laid out [channel][row][t] with the 16-byte
// chunks of each 64-byte row XOR-swizzled so that the operand reads (16 rows at one t-offset
// per pass) and the writes are free of bank conflicts.  One barrier per step.  The output
// tile goes through LDS once more, to [row][col][channel], so that the stores are 16-byte
// chunks of the channels-last layout.  The C/8 channel groups of one output tile get adjacent
// tile ids, and each XCD runs a contiguous range of ids, so the work-groups that split a pair
// row by channel run together and meet in that XCD's L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tri_mul.h"

namespace {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) bf16x8 lbf16x8;
typedef __attribute__((address_space(3))) u32x2 lu32x2;
typedef __attribute__((address_space(3))) u32x4 lu32x4;
typedef __attribute__((address_space(3))) bf16 lbf16;

constexpr int kXcd = 8;        // XCDs per MI355X; work-groups are dispatched round-robin over them
constexpr int RT = 64;         // output rows (and columns) per tile
constexpr int TT = 32;         // reduction step
constexpr int CB = 8;          // channels per work-group (one 16-byte chunk)
constexpr int kThreads = 512;  // 8 waves, one channel each
constexpr int kStage = CB * RT * TT * 2;  // bytes of one operand's stage tile (32 KiB)

// element strides (within one batch) of the row and reduction indices of P and Q, and of the
// row and column indices of the output
struct MulStrides {
  int64_t pR, pT, qR, qT, oR, oS;
};

__device__ __forceinline__ int64_t xcd_tile(int64_t ntiles) {
  const int64_t per = (ntiles + kXcd - 1) / kXcd;
  return (int64_t)(blockIdx.x % kXcd) * per + blockIdx.x / kXcd;
}

// Byte offset of (channel cc, row r, reduction t) in a stage tile: rows of 32 t (64 bytes),
// 16-byte chunk index XOR-swizzled with (r / 4) % 4.
__device__ __forceinline__ int stage_off(int cc, int r, int t) {
  return cc * (RT * TT * 2) + r * (TT * 2) + ((((t >> 3) ^ (r >> 2)) & 3) << 4) + (t & 7) * 2;
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__global__ __launch_bounds__(kThreads, 1)
void tri_mul_kernel(const bf16* __restrict__ P, const bf16* __restrict__ Q, bf16* __restrict__ out, int B, int N,
                    int C, MulStrides S) {
  __shared__ __attribute__((aligned(16))) char lds[4 * kStage];  // 2 buffers x (P, Q) = 128 KiB
  const int nT = (N + RT - 1) / RT, nCG = C / CB;
  const int64_t ntiles = (int64_t)B * nT * nT * nCG;
  const int64_t tile = xcd_tile(ntiles);
  if (tile >= ntiles) return;
  const int cg = (int)(tile % nCG);
  int64_t rest = tile / nCG;
  const int st = (int)(rest % nT); rest /= nT;
  const int rt = (int)(rest % nT);
  const int b = (int)(rest / nT);
  const int64_t base = (int64_t)b * N * N * C + cg * CB;

  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;
  // loader role: row lr of the tile, reduction quad tq (t = 4 tq .. 4 tq + 3 of the step)
  const int lr = tid >> 3, tq = tid & 7;
  const int pr = rt * RT + lr, qs = st * RT + lr;
  const bool pok = pr < N, qok = qs < N;
  const bf16* pRow = P + base + (int64_t)(pok ? pr : 0) * S.pR;
  const bf16* qRow = Q + base + (int64_t)(qok ? qs : 0) * S.qR;

  u32x4 pv[4], qv[4];
  auto load = [&](int t0) {
#pragma unroll
    for (int e = 0; e < 4; e++) {
      const int t = t0 + 4 * tq + e;
      const bool tok = t < N;
      const u32x4 z = {0u, 0u, 0u, 0u};
      pv[e] = (pok && tok) ? *(const u32x4*)(pRow + (int64_t)t * S.pT) : z;
      qv[e] = (qok && tok) ? *(const u32x4*)(qRow + (int64_t)t * S.qT) : z;
    }
  };
  // 4 chunks (t = 4tq..4tq+3) x 8 channels -> 8 channel rows of 4 t; dword d of a chunk holds
  // channels 2d (low half) and 2d + 1 (high half)
  auto store = [&](int buf) {
    char* Pt = lds + buf * 2 * kStage;
    char* Qt = Pt + kStage;
#pragma unroll
    for (int d = 0; d < 4; d++) {
      const u32x2 plo = {(pv[0][d] & 0xFFFFu) | (pv[1][d] << 16), (pv[2][d] & 0xFFFFu) | (pv[3][d] << 16)};
      const u32x2 phi = {(pv[0][d] >> 16) | (pv[1][d] & 0xFFFF0000u), (pv[2][d] >> 16) | (pv[3][d] & 0xFFFF0000u)};
      const u32x2 qlo = {(qv[0][d] & 0xFFFFu) | (qv[1][d] << 16), (qv[2][d] & 0xFFFFu) | (qv[3][d] << 16)};
      const u32x2 qhi = {(qv[0][d] >> 16) | (qv[1][d] & 0xFFFF0000u), (qv[2][d] >> 16) | (qv[3][d] & 0xFFFF0000u)};
      *(lu32x2*)(Pt + stage_off(2 * d, lr, 4 * tq)) = plo;
      *(lu32x2*)(Pt + stage_off(2 * d + 1, lr, 4 * tq)) = phi;
      *(lu32x2*)(Qt + stage_off(2 * d, lr, 4 * tq)) = qlo;
      *(lu32x2*)(Qt + stage_off(2 * d + 1, lr, 4 * tq)) = qhi;
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < 2; j++) acc[i][j] = f32x16{};

  const int nsteps = (N + TT - 1) / TT;
  load(0);
  store(0);
  __syncthreads();
  for (int s = 0; s < nsteps; s++) {
    const bool more = s + 1 < nsteps;
    if (more) load((s + 1) * TT);  // in flight while this step's products run
    const char* Pt = lds + (s & 1) * 2 * kStage;
    const char* Qt = Pt + kStage;
#pragma unroll
    for (int kk = 0; kk < 2; kk++) {
      // A operand: row l%32 (+32), reduction 16 kk + 8 (l/32) .. +7; B operand likewise
      const int t = kk * 16 + 8 * (l >> 5);
      const bf16x8 a0 = *(const lbf16x8*)(Pt + stage_off(w, l & 31, t));
      const bf16x8 a1 = *(const lbf16x8*)(Pt + stage_off(w, 32 + (l & 31), t));
      const bf16x8 b0 = *(const lbf16x8*)(Qt + stage_off(w, l & 31, t));
      const bf16x8 b1 = *(const lbf16x8*)(Qt + stage_off(w, 32 + (l & 31), t));
      acc[0][0] = mfma32(a0, b0, acc[0][0]);
      acc[0][1] = mfma32(a0, b1, acc[0][1]);
      acc[1][0] = mfma32(a1, b0, acc[1][0]);
      acc[1][1] = mfma32(a1, b1, acc[1][1]);
    }
    if (more) store((s + 1) & 1);  // that buffer's last readers passed the previous barrier
    __syncthreads();
  }

  // output tile through LDS as [row][col][channel] bf16 (64 KiB, the stage buffers' space)
  lbf16* E = (lbf16*)lds;
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < 2; j++)
#pragma unroll
      for (int e = 0; e < 16; e++) {
        const int r = i * 32 + 8 * (e >> 2) + 4 * (l >> 5) + (e & 3);
        const int c = j * 32 + (l & 31);
        E[(r * RT + c) * CB + w] = (bf16)acc[i][j][e];
      }
  __syncthreads();
  bf16* ob = out + base;
#pragma unroll
  for (int e = 0; e < RT * RT / kThreads; e++) {
    const int q = tid + e * kThreads;
    const int r = q / RT, c = q % RT;
    const int gr = rt * RT + r, gc = st * RT + c;
    if (gr < N && gc < N)
      *(u32x4*)(ob + (int64_t)gr * S.oR + (int64_t)gc * S.oS) = *(const lu32x4*)(E + q * CB);
  }
}

// ------------------------------------------------------------------ channels-first layout
// With a, b, x (and the gradients) laid out [B, C, N, N], each channel is a plain N x N matrix
// and the product of one channel is an ordinary matrix product whose operands are either
// contiguous along the reduction index t ("t-major": element (r, t) at r*N + t) or along the
// row index r ("r-major": at t*N + r).  A work-group computes a 128 x 256 output tile of one
// channel with 4 waves (64 x 128 each, eight 32x32x16 accumulator tiles: six operand reads per
// eight products), in reduction steps of
// 32 staged through a three-stage LDS ring filled by direct-to-LDS loads issued two steps
// ahead.  Loads are 16-byte chunks along the contiguous index.
// A t-major operand is stored [row][t] (64-byte rows, XOR-swizzled chunks) and read with
// ds_read_b128; an r-major operand is stored as loaded, [t][row] (rows of 256 or 512 bytes whose 64-byte
// blocks are XOR-swizzled by t % 4, so that the transposing reads of 32 lanes, 4 t-rows x 64
// bytes, hit distinct banks) and read with ds_read_b64_tr_b16, which hands each lane 4
// consecutive t of its row.  The output tile goes through LDS to leave as full 512-byte row
// segments.

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 ls16x4;

constexpr int GR = 128;          // output tile rows (P side)
constexpr int GS = 256;          // output tile columns (Q side)
constexpr int GK = 32;           // reduction step
constexpr int kGThreads = 256;   // 4 waves, 64 x 128 outputs each
constexpr int kRowT = GK * 2;    // bytes per row of a t-major stage tile

// Operand fragment for a 32x32x16 product: the 8 consecutive t (from t) of tile row `row`.
// W is the operand's tile width (rows of a t-major tile, columns of an r-major one).
template <bool TMAJ, int W>
__device__ __forceinline__ bf16x8 frag(const char* X, int row, int t, int l) {
  if (TMAJ) {
    return *(const lbf16x8*)(X + row * kRowT + ((((t >> 3) ^ (row >> 2)) & 3) << 4));
  } else {
    // lanes of a 16-lane group share (row - l%16, t); lane u addresses t-row t + u/4, column
    // row - l%16 + 4 (u%4) and receives rows t..t+3 of column row
    const int u = l & 15;
    const int tt = t + (u >> 2), cb = (row - u + 4 * (u & 3)) * 2;  // t-row, byte in the row
    const char* p = X + tt * (W * 2) + (cb ^ ((tt & 3) << 6));
    const char* p4 = X + (tt + 4) * (W * 2) + (cb ^ (((tt + 4) & 3) << 6));
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ls16x4*)p);
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ls16x4*)p4);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  }
}

// Raw buffer descriptor over [base, base + bytes): loads at or past the end return zeros.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 raw_rsrc(const void* base, int bytes) {
  const unsigned long long a = (unsigned long long)(uintptr_t)base;
  i32x4 r = {__builtin_amdgcn_readfirstlane((int)(unsigned)a),
             __builtin_amdgcn_readfirstlane((int)((unsigned)(a >> 32) & 0xFFFFu)),
             __builtin_amdgcn_readfirstlane(bytes), 0x00020000};
  return r;
}
// 16 bytes per lane from the buffer straight into LDS: lane l's bytes land at lds_wave_base + 16 l.
// The statement is invisible to the compiler's wait-count tracking: the kernel waits for these
// loads itself (vmcnt) before the barrier that publishes them.  It carries its own wait states
// (one after the M0 write, five before a load whose scalar operands a vector instruction may
// have just written).
__device__ __forceinline__ void dma16(i32x4 rsrc, unsigned voff, int soff, unsigned lds_wave_base) {
  asm volatile("s_mov_b32 m0, %3\n\ts_nop 4\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :: "v"(voff), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(soff)),
                  "s"(__builtin_amdgcn_readfirstlane(lds_wave_base)) : "memory", "m0");
}
// Barrier that orders LDS accesses only (it does not wait for the loads still in flight).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
constexpr unsigned kOob = 0x80000000u;  // a per-lane offset past any buffer: the load returns zeros

// Per-lane offsets of one operand's stage loads.  The waves issue 1 KiB loads (lane l of load i
// fills 16-byte unit u = 64 i + l of the stage tile), so each lane decides which global chunk
// lands in that unit: the swizzled layouts come from the choice of source.  t-major tile
// [W rows][4 units]: unit u is row u/4, swizzled chunk u%4; r-major tile [32 t][W/8 units]:
// unit u is t-row u/(W/8), swizzled chunk u%(W/8) (64-byte blocks XOR t%4).
struct StageLane {
  unsigned off;  // byte offset of this lane's chunk relative to the step's tile origin
  int t;         // reduction index of the chunk relative to the step (t-major only)
  bool rok;      // r-major: the chunk's columns lie inside the matrix
};
template <bool TMAJ, int W>
__device__ __forceinline__ StageLane stage_lane(int u, int N, int x0) {
  StageLane s;
  if (TMAJ) {
    const int row = u >> 2, q = (u & 3) ^ ((row >> 2) & 3);
    s.off = (unsigned)((row * N + q * 8) * 2);
    s.t = q * 8;
    s.rok = true;  // rows past N lie past the buffer's end
  } else {
    constexpr int U = W / 8;  // units per t-row
    const int t = u / U, q = (u % U) ^ ((t & 3) << 2);
    s.off = (unsigned)((t * N + q * 8) * 2);
    s.t = t;
    s.rok = x0 + q * 8 < N;
  }
  return s;
}

template <bool PT, bool QT>
__global__ __launch_bounds__(kGThreads, 2)
void tri_mul_cf_kernel(const bf16* __restrict__ P, const bf16* __restrict__ Q, bf16* __restrict__ out, int B, int N,
                       int C) {
  constexpr int kStages = 3;                       // loads run two steps ahead of the products
  constexpr int kPB = GR * GK * 2, kQB = GS * GK * 2;  // stage bytes of P (8 KiB) and Q (16 KiB)
  constexpr int kStageB = kPB + kQB;
  constexpr int LP = kPB / 1024 / 4, LQ = kQB / 1024 / 4;  // 1 KiB loads per wave and step
  __shared__ __attribute__((aligned(16))) char lds[kStages * kStageB];
  const int nR = (N + GR - 1) / GR, nS = (N + GS - 1) / GS;
  const int64_t ntiles = (int64_t)B * C * nR * nS;
  const int64_t tile = xcd_tile(ntiles);
  if (tile >= ntiles) return;
  const int st = (int)(tile % nS);
  int64_t rest = tile / nS;
  const int rt = (int)(rest % nR);
  const int64_t bc = rest / nR;  // b * C + c
  const int64_t base = bc * N * N;
  const int r0 = rt * GR, s0 = st * GS;

  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;
  const i32x4 rp = raw_rsrc(P + base, N * N * 2), rq = raw_rsrc(Q + base, N * N * 2);
  const unsigned lds0 = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)(const __attribute__((address_space(3))) char*)lds);
  StageLane lp[LP], lq[LQ];
#pragma unroll
  for (int e = 0; e < LP; e++) lp[e] = stage_lane<PT, GR>((LP * w + e) * 64 + l, N, r0);
#pragma unroll
  for (int e = 0; e < LQ; e++) lq[e] = stage_lane<QT, GS>((LQ * w + e) * 64 + l, N, s0);
  // issue the loads of reduction step s into stage buffer s % 3
  auto issue = [&](int s) {
    const int t0 = s * GK;
    const unsigned dst = lds0 + (s % kStages) * kStageB;
    // tile origin: (row x0, t0) of a t-major operand, (t-row t0, column x0) of an r-major one
    const int sp = PT ? (r0 * N + t0) * 2 : (t0 * N + r0) * 2;
    const int sq = QT ? (s0 * N + t0) * 2 : (t0 * N + s0) * 2;
#pragma unroll
    for (int e = 0; e < LP; e++) {
      const bool ok = PT ? t0 + lp[e].t < N : lp[e].rok;
      dma16(rp, ok ? lp[e].off : kOob, sp, dst + (LP * w + e) * 1024);
    }
#pragma unroll
    for (int e = 0; e < LQ; e++) {
      const bool ok = QT ? t0 + lq[e].t < N : lq[e].rok;
      dma16(rq, ok ? lq[e].off : kOob, sq, dst + kPB + (LQ * w + e) * 1024);
    }
  };

  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) acc[i][j] = f32x16{};
  const int wr = (w >> 1) * 64, wc = (w & 1) * 128;  // this wave's 64 x 128 sub-tile

  const int nsteps = (N + GK - 1) / GK;
  issue(0);
  if (nsteps > 1) issue(1);
  if (nsteps > 1) __builtin_amdgcn_s_waitcnt(0x0F70 | (LP + LQ));  // step 0's loads have landed
  else __builtin_amdgcn_s_waitcnt(0x0F70);
  lds_barrier();
  for (int s = 0; s < nsteps; s++) {
    // stage (s+2) % 3 was last read in step s-1, which every wave finished before the barrier
    if (s + 2 < nsteps) issue(s + 2);
    const char* Pt = lds + (s % kStages) * kStageB;
    const char* Qt = Pt + kPB;
#pragma unroll
    for (int kk = 0; kk < 2; kk++) {
      const int t = kk * 16 + 8 * (l >> 5);
      bf16x8 a[2], bq[4];
#pragma unroll
      for (int i = 0; i < 2; i++) a[i] = frag<PT, GR>(Pt, wr + 32 * i + (l & 31), t, l);
#pragma unroll
      for (int j = 0; j < 4; j++) bq[j] = frag<QT, GS>(Qt, wc + 32 * j + (l & 31), t, l);
#pragma unroll
      for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) acc[i][j] = mfma32(a[i], bq[j], acc[i][j]);
    }
    // step s+1's loads have landed for this wave once only step s+2's (if issued) are pending
    if (s + 2 < nsteps) __builtin_amdgcn_s_waitcnt(0x0F70 | (LP + LQ));
    else __builtin_amdgcn_s_waitcnt(0x0F70);
    lds_barrier();
  }

  // output tile through LDS: [128 rows][256 columns] bf16 (64 KiB; no load is in flight)
  lbf16* E = (lbf16*)lds;
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
      for (int e = 0; e < 16; e++) {
        const int r = wr + i * 32 + 8 * (e >> 2) + 4 * (l >> 5) + (e & 3);
        const int c = wc + j * 32 + (l & 31);
        E[r * GS + c] = (bf16)acc[i][j][e];
      }
  __syncthreads();
  bf16* oc = out + base;
#pragma unroll
  for (int e = 0; e < GR * GS / 8 / kGThreads; e++) {
    const int ch = tid + e * kGThreads;
    const int r = ch / (GS / 8), c = (ch % (GS / 8)) * 8;
    if (r0 + r < N && s0 + c < N) *(u32x4*)(oc + (int64_t)(r0 + r) * N + s0 + c) = *(const lu32x4*)(E + r * GS + c);
  }
}

// ------------------------------------------------------------------ layout change
// out[b][k][r] = in[b][r][k] for an R x K bf16 matrix per batch (R and K multiples of 8):
// channels last -> channels first with (R, K) = (N*N, C), and back with (C, N*N).  A work-group
// moves a 64 x 64 tile through LDS: 16-byte loads along k, then each thread gathers 8
// consecutive r of one k from LDS and stores them as one 16-byte chunk, so that both sides are
// runs of whole 128-byte segments.
constexpr int TP = 64;
constexpr int TPS = TP + 8;  // LDS row stride (elements): 144-byte rows keep the chunks aligned
__global__ __launch_bounds__(256)
void transpose_kernel(const bf16* __restrict__ in, bf16* __restrict__ out, int64_t R, int64_t K, int64_t tilesR,
                      int64_t tilesK) {
  __shared__ __attribute__((aligned(16))) unsigned short T[TP * TPS];
  const int64_t per = tilesR * tilesK;
  const int64_t b = blockIdx.x / per, rem = blockIdx.x % per;
  const int64_t r0 = (rem / tilesK) * TP, k0 = (rem % tilesK) * TP;
  const unsigned short* src = (const unsigned short*)in + b * R * K;
  unsigned short* dst = (unsigned short*)out + b * R * K;
  const int tid = threadIdx.x;
#pragma unroll
  for (int e = 0; e < 2; e++) {  // chunk (row r, k-chunk kc): 8 threads per 128-byte row segment
    const int ch = tid + e * 256, r = ch >> 3, kc = ch & 7;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r0 + r < R && k0 + kc * 8 < K) v = *(const u32x4*)(src + (r0 + r) * K + k0 + kc * 8);
    *(__attribute__((address_space(3))) u32x4*)(T + r * TPS + kc * 8) = v;
  }
  __syncthreads();
#pragma unroll
  for (int e = 0; e < 2; e++) {  // output chunk (row k, r-chunk rc)
    const int ch = tid + e * 256, k = ch >> 3, rc = ch & 7;
    if (k0 + k < K && r0 + rc * 8 < R) {
      unsigned w[4];
#pragma unroll
      for (int i = 0; i < 4; i++)
        w[i] = (unsigned)T[(rc * 8 + 2 * i) * TPS + k] | ((unsigned)T[(rc * 8 + 2 * i + 1) * TPS + k] << 16);
      const u32x4 v = {w[0], w[1], w[2], w[3]};
      *(u32x4*)(dst + (k0 + k) * R + r0 + rc * 8) = v;
    }
  }
}

// ------------------------------------------------------------------ input gating
// a = sigmoid(g) * p * mask[position] in FP32, rounded once to bf16; g and p channels last
// [B][N*N][C].  With CF the result leaves channels first [B][C][N*N] through a 64 x 64 LDS tile
// (positions x channels), like the layout change, so that gating and layout change cost one
// pass over HBM.  The backward reads da in the same layout and writes dg, dp channels last:
//   dp = da * m * sigmoid(g),   dg = da * m * p * sigmoid(g) (1 - sigmoid(g)).
__device__ __forceinline__ float bf_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(unsigned w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ unsigned pack_bf16(float lo, float hi) {
  const bf16 l = (bf16)lo, h = (bf16)hi;
  return (unsigned)__builtin_bit_cast(unsigned short, l) | ((unsigned)__builtin_bit_cast(unsigned short, h) << 16);
}
__device__ __forceinline__ float sigmoid_f32(float x) {
  return 1.0f / (1.0f + __builtin_amdgcn_exp2f(-x * 1.4426950408889634f));
}

template <bool CF>
__global__ __launch_bounds__(256)
void gate_fwd_kernel(const bf16* __restrict__ g, const bf16* __restrict__ p, const uint8_t* __restrict__ mask,
                     bf16* __restrict__ a, int64_t R, int64_t K, int64_t tilesR, int64_t tilesK) {
  __shared__ __attribute__((aligned(16))) unsigned short T[TP * TPS];
  const int64_t per = tilesR * tilesK;
  const int64_t b = blockIdx.x / per, rem = blockIdx.x % per;
  const int64_t r0 = (rem / tilesK) * TP, k0 = (rem % tilesK) * TP;
  const int64_t base = b * R * K;
  const int tid = threadIdx.x;
#pragma unroll
  for (int e = 0; e < 2; e++) {  // chunk (position r, channels kc*8..+7)
    const int ch = tid + e * 256, r = ch >> 3, kc = ch & 7;
    u32x4 out = {0u, 0u, 0u, 0u};
    const bool ok = r0 + r < R && k0 + kc * 8 < K;
    if (ok) {
      const int64_t off = base + (r0 + r) * K + k0 + kc * 8;
      const u32x4 gv = *(const u32x4*)(g + off), pv = *(const u32x4*)(p + off);
      const float m = (mask && mask[b * R + r0 + r] == 0) ? 0.0f : 1.0f;
#pragma unroll
      for (int d = 0; d < 4; d++)
        out[d] = pack_bf16(sigmoid_f32(bf_lo(gv[d])) * bf_lo(pv[d]) * m, sigmoid_f32(bf_hi(gv[d])) * bf_hi(pv[d]) * m);
      if (!CF) *(u32x4*)(a + off) = out;
    }
    if (CF) *(__attribute__((address_space(3))) u32x4*)(T + r * TPS + kc * 8) = out;
  }
  if (!CF) return;
  __syncthreads();
  unsigned short* dst = (unsigned short*)a + base;
#pragma unroll
  for (int e = 0; e < 2; e++) {  // output chunk (channel k, positions rc*8..+7)
    const int ch = tid + e * 256, k = ch >> 3, rc = ch & 7;
    if (k0 + k < K && r0 + rc * 8 < R) {
      unsigned w[4];
#pragma unroll
      for (int i = 0; i < 4; i++)
        w[i] = (unsigned)T[(rc * 8 + 2 * i) * TPS + k] | ((unsigned)T[(rc * 8 + 2 * i + 1) * TPS + k] << 16);
      const u32x4 v = {w[0], w[1], w[2], w[3]};
      *(u32x4*)(dst + (k0 + k) * R + r0 + rc * 8) = v;
    }
  }
}

template <bool CF>
__global__ __launch_bounds__(256)
void gate_bwd_kernel(const bf16* __restrict__ g, const bf16* __restrict__ p, const uint8_t* __restrict__ mask,
                     const bf16* __restrict__ da, bf16* __restrict__ dg, bf16* __restrict__ dp, int64_t R, int64_t K,
                     int64_t tilesR, int64_t tilesK) {
  __shared__ __attribute__((aligned(16))) unsigned short T[TP * TPS];
  const int64_t per = tilesR * tilesK;
  const int64_t b = blockIdx.x / per, rem = blockIdx.x % per;
  const int64_t r0 = (rem / tilesK) * TP, k0 = (rem % tilesK) * TP;
  const int64_t base = b * R * K;
  const int tid = threadIdx.x;
  if (CF) {  // da channels first: chunks (channel k, 8 positions) into T[position][channel]
#pragma unroll
    for (int e = 0; e < 2; e++) {
      const int ch = tid + e * 256, k = ch >> 3, rc = ch & 7;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (k0 + k < K && r0 + rc * 8 < R) v = *(const u32x4*)(da + base + (k0 + k) * R + r0 + rc * 8);
#pragma unroll
      for (int i = 0; i < 4; i++) {
        T[(rc * 8 + 2 * i) * TPS + k] = (unsigned short)(v[i] & 0xFFFFu);
        T[(rc * 8 + 2 * i + 1) * TPS + k] = (unsigned short)(v[i] >> 16);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int e = 0; e < 2; e++) {  // chunk (position r, channels kc*8..+7)
    const int ch = tid + e * 256, r = ch >> 3, kc = ch & 7;
    if (r0 + r < R && k0 + kc * 8 < K) {
      const int64_t off = base + (r0 + r) * K + k0 + kc * 8;
      const u32x4 gv = *(const u32x4*)(g + off), pv = *(const u32x4*)(p + off);
      const u32x4 dv = CF ? *(const __attribute__((address_space(3))) u32x4*)(T + r * TPS + kc * 8)
                          : *(const u32x4*)(da + off);
      const float m = (mask && mask[b * R + r0 + r] == 0) ? 0.0f : 1.0f;
      u32x4 og, op;
#pragma unroll
      for (int d = 0; d < 4; d++) {
        const float s0 = sigmoid_f32(bf_lo(gv[d])), s1 = sigmoid_f32(bf_hi(gv[d]));
        const float d0 = bf_lo(dv[d]) * m, d1 = bf_hi(dv[d]) * m;
        op[d] = pack_bf16(d0 * s0, d1 * s1);
        og[d] = pack_bf16(d0 * bf_lo(pv[d]) * (s0 * (1.0f - s0)), d1 * bf_hi(pv[d]) * (s1 * (1.0f - s1)));
      }
      *(u32x4*)(dg + off) = og;
      *(u32x4*)(dp + off) = op;
    }
  }
}

void transpose(const void* in, void* out, int64_t B, int64_t R, int64_t K, hipStream_t st) {
  const int64_t tr = (R + TP - 1) / TP, tk = (K + TP - 1) / TP;
  hipLaunchKernelGGL(transpose_kernel, dim3((unsigned)(B * tr * tk)), dim3(256), 0, st, (const bf16*)in, (bf16*)out,
                     R, K, tr, tk);
}

unsigned grid_xcd(int64_t ntiles) { return (unsigned)((ntiles + kXcd - 1) / kXcd * kXcd); }

struct Range { const void* p; int64_t n; };
constexpr int64_t kWsAlign = 256;
int64_t ws_tensor_bytes(int64_t B, int64_t N, int64_t C) { return (B * N * N * C * 2 + kWsAlign - 1) / kWsAlign * kWsAlign; }
bool overlap(Range x, Range y) {
  const uintptr_t a0 = (uintptr_t)x.p, a1 = a0 + (uintptr_t)x.n, b0 = (uintptr_t)y.p, b1 = b0 + (uintptr_t)y.n;
  return a0 < b1 && b0 < a1;
}
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

tri_attn_status check_shape(int direction, int layout, int64_t B, int64_t N, int64_t C) {
  if (direction != TRI_MUL_OUTGOING && direction != TRI_MUL_INCOMING) return TRI_ATTN_ERROR_INVALID_VALUE;
  if (layout != TRI_MUL_CHANNELS_LAST && layout != TRI_MUL_CHANNELS_FIRST) return TRI_ATTN_ERROR_INVALID_VALUE;
  if (B < 1 || N < 1 || C < 1) return TRI_ATTN_ERROR_INVALID_VALUE;
  if (C > 1024 || N > TRI_MUL_MAX_N || B > (1 << 16)) return TRI_ATTN_ERROR_UNSUPPORTED;
  if (layout == TRI_MUL_CHANNELS_LAST && C % CB != 0) return TRI_ATTN_ERROR_UNSUPPORTED;
  if (layout == TRI_MUL_CHANNELS_FIRST && N % 8 != 0) return TRI_ATTN_ERROR_UNSUPPORTED;
  return TRI_ATTN_SUCCESS;
}

tri_attn_status launch(const void* p, const void* q, void* o, int64_t B, int64_t N, int64_t C, MulStrides S,
                       hipStream_t st) {
  const int64_t nT = (N + RT - 1) / RT;
  const int64_t ntiles = B * nT * nT * (C / CB);
  hipLaunchKernelGGL(tri_mul_kernel, dim3(grid_xcd(ntiles)), dim3(kThreads), 0, st, (const bf16*)p, (const bf16*)q,
                     (bf16*)o, (int)B, (int)N, (int)C, S);
  return hipGetLastError() == hipSuccess ? TRI_ATTN_SUCCESS : TRI_ATTN_ERROR_LAUNCH;
}

// channels-first: OUT_c = P_c-product-Q_c with P, Q t-major (PT, QT) or r-major
tri_attn_status launch_cf(bool pt, bool qt, const void* p, const void* q, void* o, int64_t B, int64_t N, int64_t C,
                          hipStream_t st) {
  const dim3 grid(grid_xcd(B * C * ((N + GR - 1) / GR) * ((N + GS - 1) / GS))), block(kGThreads);
  const bf16 *P = (const bf16*)p, *Q = (const bf16*)q;
  bf16* O = (bf16*)o;
  if (pt && qt) hipLaunchKernelGGL((tri_mul_cf_kernel<true, true>), grid, block, 0, st, P, Q, O, (int)B, (int)N, (int)C);
  else if (pt) hipLaunchKernelGGL((tri_mul_cf_kernel<true, false>), grid, block, 0, st, P, Q, O, (int)B, (int)N, (int)C);
  else if (qt) hipLaunchKernelGGL((tri_mul_cf_kernel<false, true>), grid, block, 0, st, P, Q, O, (int)B, (int)N, (int)C);
  else hipLaunchKernelGGL((tri_mul_cf_kernel<false, false>), grid, block, 0, st, P, Q, O, (int)B, (int)N, (int)C);
  return hipGetLastError() == hipSuccess ? TRI_ATTN_SUCCESS : TRI_ATTN_ERROR_LAUNCH;
}

}  // namespace

extern "C" {

size_t tri_mul_workspace_bytes(int layout, int64_t B, int64_t N, int64_t C) {
  if (check_shape(TRI_MUL_OUTGOING, layout, B, N, C) != TRI_ATTN_SUCCESS) return 0;
  if (layout == TRI_MUL_CHANNELS_FIRST || N % 8 != 0) return 0;
  return (size_t)(5 * ws_tensor_bytes(B, N, C));  // the backward's a, b, dx, da, db channels first
}

tri_attn_status tri_mul_fwd(int direction, int layout, int64_t B, int64_t N, int64_t C, const void* a, const void* b,
                            void* x, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const tri_attn_status st = check_shape(direction, layout, B, N, C);
  if (st != TRI_ATTN_SUCCESS) return st;
  if (!a || !b || !x) return TRI_ATTN_ERROR_INVALID_VALUE;
  const int64_t bytes = B * N * N * C * 2;
  if (overlap({x, bytes}, {a, bytes}) || overlap({x, bytes}, {b, bytes})) return TRI_ATTN_ERROR_INVALID_VALUE;
  const Range ws{workspace, (int64_t)workspace_bytes};
  if (workspace && (overlap(ws, {a, bytes}) || overlap(ws, {b, bytes}) || overlap(ws, {x, bytes})))
    return TRI_ATTN_ERROR_INVALID_VALUE;
  if (!aligned16(a) || !aligned16(b) || !aligned16(x) || (workspace && !aligned16(workspace)))
    return TRI_ATTN_ERROR_MISALIGNED;
  if (layout == TRI_MUL_CHANNELS_FIRST)  // outgoing: a, b t-major; incoming: both r-major
    return direction == TRI_MUL_OUTGOING ? launch_cf(true, true, a, b, x, B, N, C, stream)
                                         : launch_cf(false, false, a, b, x, B, N, C, stream);
  if (workspace && N % 8 == 0) {  // channels last through the workspace: change layout, run the channels-first product
    if (workspace_bytes < tri_mul_workspace_bytes(layout, B, N, C)) return TRI_ATTN_ERROR_WORKSPACE;
    const int64_t tb = ws_tensor_bytes(B, N, C);
    char* w = (char*)workspace;
    transpose(a, w, B, N * N, C, stream);
    transpose(b, w + tb, B, N * N, C, stream);
    const tri_attn_status r = direction == TRI_MUL_OUTGOING ? launch_cf(true, true, w, w + tb, w + 2 * tb, B, N, C, stream)
                                                            : launch_cf(false, false, w, w + tb, w + 2 * tb, B, N, C, stream);
    if (r != TRI_ATTN_SUCCESS) return r;
    transpose(w + 2 * tb, x, B, C, N * N, stream);
    return hipGetLastError() == hipSuccess ? TRI_ATTN_SUCCESS : TRI_ATTN_ERROR_LAUNCH;
  }
  const int64_t NC = N * C;
  // outgoing: P[r=i,t=k] = a[i,k], Q[s=j,t=k] = b[j,k]; incoming: P[r=i,t=k] = a[k,i], Q = b[k,j]
  const MulStrides S = direction == TRI_MUL_OUTGOING ? MulStrides{NC, C, NC, C, NC, C}
                                                     : MulStrides{C, NC, C, NC, NC, C};
  return launch(a, b, x, B, N, C, S, stream);
}

tri_attn_status tri_mul_bwd(int direction, int layout, int64_t B, int64_t N, int64_t C, const void* a,
                            const void* b, const void* dx, void* da, void* db, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  const tri_attn_status st = check_shape(direction, layout, B, N, C);
  if (st != TRI_ATTN_SUCCESS) return st;
  if (!a || !b || !dx || !da || !db) return TRI_ATTN_ERROR_INVALID_VALUE;
  const int64_t bytes = B * N * N * C * 2;
  const Range ins[] = {{a, bytes}, {b, bytes}, {dx, bytes}};
  for (const Range& r : ins)
    if (overlap({da, bytes}, r) || overlap({db, bytes}, r)) return TRI_ATTN_ERROR_INVALID_VALUE;
  if (overlap({da, bytes}, {db, bytes})) return TRI_ATTN_ERROR_INVALID_VALUE;
  const Range ws{workspace, (int64_t)workspace_bytes};
  if (workspace) {
    const Range all[] = {{a, bytes}, {b, bytes}, {dx, bytes}, {da, bytes}, {db, bytes}};
    for (const Range& r : all)
      if (overlap(ws, r)) return TRI_ATTN_ERROR_INVALID_VALUE;
  }
  if (!aligned16(a) || !aligned16(b) || !aligned16(dx) || !aligned16(da) || !aligned16(db) ||
      (workspace && !aligned16(workspace)))
    return TRI_ATTN_ERROR_MISALIGNED;
  const int64_t NC = N * C;
  tri_attn_status r1, r2;
  auto cf_pair = [&](const void* A, const void* Bv, const void* DX, void* DA, void* DB) {
    if (direction == TRI_MUL_OUTGOING) {
      r1 = launch_cf(true, false, DX, Bv, DA, B, N, C, stream);   // da[i,k] = sum_j dx[i,j] b[j,k]
      r2 = launch_cf(false, false, DX, A, DB, B, N, C, stream);   // db[j,k] = sum_i dx[i,j] a[i,k]
    } else {
      r1 = launch_cf(true, true, Bv, DX, DA, B, N, C, stream);    // da[k,i] = sum_j b[k,j] dx[i,j]
      r2 = launch_cf(true, false, A, DX, DB, B, N, C, stream);    // db[k,j] = sum_i a[k,i] dx[i,j]
    }
  };
  if (layout == TRI_MUL_CHANNELS_FIRST) {
    cf_pair(a, b, dx, da, db);
    return r1 != TRI_ATTN_SUCCESS ? r1 : r2;
  }
  if (workspace && N % 8 == 0) {  // channels last through the workspace
    if (workspace_bytes < tri_mul_workspace_bytes(layout, B, N, C)) return TRI_ATTN_ERROR_WORKSPACE;
    const int64_t tb = ws_tensor_bytes(B, N, C);
    char* w = (char*)workspace;
    transpose(a, w, B, N * N, C, stream);
    transpose(b, w + tb, B, N * N, C, stream);
    transpose(dx, w + 2 * tb, B, N * N, C, stream);
    cf_pair(w, w + tb, w + 2 * tb, w + 3 * tb, w + 4 * tb);
    if (r1 != TRI_ATTN_SUCCESS || r2 != TRI_ATTN_SUCCESS) return r1 != TRI_ATTN_SUCCESS ? r1 : r2;
    transpose(w + 3 * tb, da, B, C, N * N, stream);
    transpose(w + 4 * tb, db, B, C, N * N, stream);
    return hipGetLastError() == hipSuccess ? TRI_ATTN_SUCCESS : TRI_ATTN_ERROR_LAUNCH;
  }
  if (direction == TRI_MUL_OUTGOING) {
    // da[i,k] = sum_j dx[i,j] b[j,k]: P[r=i,t=j] = dx[i,j], Q[s=k,t=j] = b[j,k]
    r1 = launch(dx, b, da, B, N, C, MulStrides{NC, C, C, NC, NC, C}, stream);
    // db[j,k] = sum_i dx[i,j] a[i,k]: P[r=j,t=i] = dx[i,j], Q[s=k,t=i] = a[i,k]
    r2 = launch(dx, a, db, B, N, C, MulStrides{C, NC, C, NC, NC, C}, stream);
  } else {
    // da[k,i] = sum_j b[k,j] dx[i,j]: P[r=k,t=j] = b[k,j], Q[s=i,t=j] = dx[i,j]
    r1 = launch(b, dx, da, B, N, C, MulStrides{NC, C, NC, C, NC, C}, stream);
    // db[k,j] = sum_i a[k,i] dx[i,j]: P[r=k,t=i] = a[k,i], Q[s=j,t=i] = dx[i,j]
    r2 = launch(a, dx, db, B, N, C, MulStrides{NC, C, C, NC, NC, C}, stream);
  }
  return r1 != TRI_ATTN_SUCCESS ? r1 : r2;
}

tri_attn_status tri_mul_gate_fwd(int layout, int64_t B, int64_t N, int64_t C, const void* g, const void* p,
                                 const uint8_t* mask, void* a, hipStream_t stream) {
  if (layout != TRI_MUL_CHANNELS_LAST && layout != TRI_MUL_CHANNELS_FIRST) return TRI_ATTN_ERROR_INVALID_VALUE;
  if (B < 1 || N < 1 || C < 1 || !g || !p || !a) return TRI_ATTN_ERROR_INVALID_VALUE;
  if (C % 8 != 0 || C > 1024 || N > TRI_MUL_MAX_N || B > (1 << 16) ||
      (layout == TRI_MUL_CHANNELS_FIRST && N % 8 != 0))
    return TRI_ATTN_ERROR_UNSUPPORTED;
  const int64_t bytes = B * N * N * C * 2;
  if (overlap({a, bytes}, {g, bytes}) || overlap({a, bytes}, {p, bytes}) ||
      (mask && overlap({a, bytes}, {mask, B * N * N})))
    return TRI_ATTN_ERROR_INVALID_VALUE;
  if (!aligned16(g) || !aligned16(p) || !aligned16(a)) return TRI_ATTN_ERROR_MISALIGNED;
  const int64_t R = N * N, tr = (R + TP - 1) / TP, tk = (C + TP - 1) / TP;
  if (layout == TRI_MUL_CHANNELS_FIRST)
    hipLaunchKernelGGL(gate_fwd_kernel<true>, dim3((unsigned)(B * tr * tk)), dim3(256), 0, stream, (const bf16*)g,
                       (const bf16*)p, mask, (bf16*)a, R, C, tr, tk);
  else
    hipLaunchKernelGGL(gate_fwd_kernel<false>, dim3((unsigned)(B * tr * tk)), dim3(256), 0, stream, (const bf16*)g,
                       (const bf16*)p, mask, (bf16*)a, R, C, tr, tk);
  return hipGetLastError() == hipSuccess ? TRI_ATTN_SUCCESS : TRI_ATTN_ERROR_LAUNCH;
}

tri_attn_status tri_mul_gate_bwd(int layout, int64_t B, int64_t N, int64_t C, const void* g, const void* p,
                                 const uint8_t* mask, const void* da, void* dg, void* dp, hipStream_t stream) {
  if (layout != TRI_MUL_CHANNELS_LAST && layout != TRI_MUL_CHANNELS_FIRST) return TRI_ATTN_ERROR_INVALID_VALUE;
  if (B < 1 || N < 1 || C < 1 || !g || !p || !da || !dg || !dp) return TRI_ATTN_ERROR_INVALID_VALUE;
  if (C % 8 != 0 || C > 1024 || N > TRI_MUL_MAX_N || B > (1 << 16) ||
      (layout == TRI_MUL_CHANNELS_FIRST && N % 8 != 0))
    return TRI_ATTN_ERROR_UNSUPPORTED;
  const int64_t bytes = B * N * N * C * 2;
  const Range ins[] = {{g, bytes}, {p, bytes}, {da, bytes}, {mask, mask ? B * N * N : 0}};
  for (const Range& r : ins)
    if (r.p && (overlap({dg, bytes}, r) || overlap({dp, bytes}, r))) return TRI_ATTN_ERROR_INVALID_VALUE;
  if (overlap({dg, bytes}, {dp, bytes})) return TRI_ATTN_ERROR_INVALID_VALUE;
  if (!aligned16(g) || !aligned16(p) || !aligned16(da) || !aligned16(dg) || !aligned16(dp))
    return TRI_ATTN_ERROR_MISALIGNED;
  const int64_t R = N * N, tr = (R + TP - 1) / TP, tk = (C + TP - 1) / TP;
  if (layout == TRI_MUL_CHANNELS_FIRST)
    hipLaunchKernelGGL(gate_bwd_kernel<true>, dim3((unsigned)(B * tr * tk)), dim3(256), 0, stream, (const bf16*)g,
                       (const bf16*)p, mask, (const bf16*)da, (bf16*)dg, (bf16*)dp, R, C, tr, tk);
  else
    hipLaunchKernelGGL(gate_bwd_kernel<false>, dim3((unsigned)(B * tr * tk)), dim3(256), 0, stream, (const bf16*)g,
                       (const bf16*)p, mask, (const bf16*)da, (bf16*)dg, (bf16*)dp, R, C, tr, tk);
  return hipGetLastError() == hipSuccess ? TRI_ATTN_SUCCESS : TRI_ATTN_ERROR_LAUNCH;
}

}  // extern "C"
