// fused_ru.hip -- one residual unit in one kernel:
//   h <- h + conv2(Snake2(conv1_d(S) + b1)) + b2,   S = Snake1(h) (operand dtype)
// (residual unit of the DAV decoder, minimaxmusic.cpp ARCHITECTURE "Flow VAE":
// snake1 -> conv1 k=7 at dilation d -> snake2 -> conv2 k=1 -> add the skip).
//
// A workgroup owns BN frames of one row and all C channels, so the
// intermediate U = Snake2(conv1 + b1) never leaves the CU:
//   stage 1  conv1 as an implicit GEMM (M = C, K = 7 C) from the X tile
//            [n0 - 3d, n0 + BN + 3d) and the weight rows of a group of taps,
//            both staged in LDS per 64-byte channel chunk;
//   epilogue bias + Snake2, U written into LDS over the stage-1 staging area
//            (the same 64-byte chunk rows the GEMM reads);
//   stage 2  conv2 as a GEMM (M = C, K = C) from U in LDS and conv2 weight
//            chunks streamed into LDS;
//   epilogue bias, residual add, the next layer's Snake operand if one is
//            asked for (for the last unit: the head's Snake applied to the
//            stored h).
// Compared with separate conv1 and conv2 launches this removes the U round
// trip through HBM (2 x C x T operands per unit) and the second launch.
//
// Operand source (template flag XH):
//   XH = false  S is an operand tensor written by the producer's epilogue,
//               and h is updated in place;
//   XH = true   S = Snake1(h_in) is computed here while the X tile is staged
//               from the residual stream, and the result goes to a
//               second buffer h (tiles read neighbouring frames of h_in, so
//               the update cannot be in place).  The producer then writes no
//               operand tensor: per channel-frame the unit moves 2 x 4 (fp32)
//               or 2 x 2 (fp16) bytes of h
//               (read + write) instead of h plus two operand passes, and the
//               residual rows of each channel chunk are read right after that
//               chunk's X tile, from lines the X loads have just brought into
//               the L2.  Snake1 gives bit-identical operands either way.
#include "internal.h"
#include "device_math.h"
#include "gemm_common.h"

namespace voc {

// Largest accumulator tile (m-blocks x n-blocks per wave) whose residual rows
// are held in registers from their chunk's X load to the final epilogue.
#ifndef VOC_RU_CHUNK_H_MAX
#define VOC_RU_CHUNK_H_MAX 8
#endif


// Eight-wave instances (one workgroup per CU) stage stage 1 through two LDS
// buffers: the next tap group (and channel chunk) is stored while the
// current one is multiplied, with one barrier per group instead of two.
#ifndef VOC_RU_DB
#define VOC_RU_DB 1
#endif
// With two buffers, the waves of the workgroup's second half multiply first
// and stage second, the first half the other way round, so that the two
// waves a SIMD holds are in opposite halves of each group's work.
#ifndef VOC_RU_PINGPONG
#define VOC_RU_PINGPONG 1
#endif

// MINB: waves per SIMD the register allocator must leave room for (the
// launch bound's second argument); for a four-wave workgroup that is the
// number of workgroups per CU.  TERMS = 2 (bf16): two-term operands (hi and
// lo planes, see bf16_lo4): the conv1 and conv2 reductions run over 2 x C
// channels, the low-term channels meeting a second copy of each weight
// chunk, and the operand written for a consumer holds both terms.
template <int OP, int WMB, int WNB, int WAVES_M, int WAVES_N, int TG, bool XH, int MINB, int TERMS>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N, MINB)
void res_unit_kernel(const ResUnitArgs a) {
  constexpr int NTH = 64 * WAVES_M * WAVES_N;  // threads per workgroup
  constexpr int CH = OpT<OP>::CH;
  constexpr int ES = OpT<OP>::ES;
  constexpr int C = WAVES_M * WMB * 16;
  constexpr int BN = WAVES_N * WNB * 16;
  constexpr int XROWS = (BN + 54 + 15) / 16 * 16;
  constexpr int NG = (7 + TG - 1) / TG;        // tap groups per channel chunk
  constexpr int WROWS = TG * C;
  constexpr int NCH = C / CH;                  // channel chunks
  constexpr int KCH = TERMS * NCH;             // reduction chunks (the low terms after the high)
  constexpr int HO = TERMS == 2 ? OP_F32 : OP;  // residual-stream element type (fp32 with two terms)
  // Eight-wave instances at two workgroups per CU (MINB 4) keep one buffer
  // and no held residual rows: their registers must fit 128 VGPRs.
  constexpr bool kTwoWG8 = WAVES_M * WAVES_N == 8 && MINB > 2;
  constexpr bool kDB = VOC_RU_DB && WAVES_M * WAVES_N == 8 && !kTwoWG8;
  constexpr int NB = kDB ? 2 : 1;              // stage-1 LDS buffers
  // Two terms with X staged from h: each channel chunk's X tile is staged
  // once as a high-term and a low-term tile, and each weight group meets
  // both (the loop runs over the NCH channel chunks); from an operand
  // tensor the low terms are further chunks (KCH of them).
  constexpr bool kPair = TERMS == 2 && XH;
  constexpr int XT = kPair ? 2 * XROWS : XROWS;  // X rows per stage-1 buffer
  constexpr int LCH = kPair ? NCH : KCH;         // stage-1 chunk steps
  constexpr int S1 = NB * (XT + WROWS) * kRowBytes;
  constexpr int UB = KCH * BN * kRowBytes;     // U tile: [KCH][BN] rows
  constexpr int S2 = UB + C * kRowBytes;
  constexpr int LDS_T = S1 > S2 ? S1 : S2;
  constexpr int LDS = LDS_T + (XH ? 2 * C * 4 : 0);  // + Snake1 parameters
  constexpr int XU = (XROWS * 4 + NTH - 1) / NTH;
  constexpr int WU = (WROWS * 4 + NTH - 1) / NTH;
  constexpr int W2U = (C * 4 + NTH - 1) / NTH;
  static_assert(WAVES_M * WAVES_N == 4 || WAVES_M * WAVES_N == 8, "four or eight waves");
  static_assert(C % CH == 0 && C % 16 == 0, "whole channel chunks");
  __shared__ __attribute__((aligned(16))) unsigned char smem[LDS];
  // Stage-1 buffers: X tiles [NB][XT], then weight groups [NB][WROWS].
  unsigned char* Xs = smem;
  unsigned char* Ws = smem + NB * XT * kRowBytes;
  unsigned char* Us = smem;          // stage 2 (after stage 1 is done)
  unsigned char* W2s = smem + UB;

  const int tid = threadIdx.x;
  const int L = xcd_remap(blockIdx.x, a.n_tiles * a.rows);
  const int n_tile = L % a.n_tiles;
  const int row = L / a.n_tiles;
  const int n0 = n_tile * BN;
  const int len = a.row_len[row];
  const int Lv = min(len * a.rate, a.T);
  if (n0 >= Lv) return;

  const int d = a.dil;
  const int xrows = BN + 6 * d;
  const int tfirst = n0 - a.pad;  // tap j reads frame n + j*d - pad
  const unsigned char* xrow = static_cast<const unsigned char*>(a.x) +
                              static_cast<int64_t>(row) * TERMS * C * a.T * ES;
  const int64_t xplane = static_cast<int64_t>(a.T) * kChunkBytes;
  const unsigned char* w1 = static_cast<const unsigned char*>(a.w1);
  const unsigned char* w2 = static_cast<const unsigned char*>(a.w2);

  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave % WAVES_M, wn = wave / WAVES_M;
  const int lr = lane & 15, lg = lane >> 4;

  f4 acc[WMB][WNB];
#pragma unroll
  for (int i = 0; i < WMB; ++i)
#pragma unroll
    for (int j = 0; j < WNB; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};

  // The residual h of this tile is read into registers early, so its HBM
  // latency overlaps the GEMM stages instead of stalling the final epilogue:
  // at kernel start for small tiles, after stage 1 otherwise.
  // With XH the rows of each channel chunk are read right after its X tile
  // instead (see load_x), register room permitting.
  constexpr bool kEarlyH = !XH && WMB * WNB <= 8;
  constexpr bool kChunkH = XH && WMB * WNB <= VOC_RU_CHUNK_H_MAX && !kTwoWG8;
  typename HQuad<HO>::T hres[WMB][WNB];  // converted in the final epilogue
  auto load_h_block = [&](int mb) {
    const int m = wm * WMB * 16 + mb * 16 + lg * 4;
    const int64_t hbase = (static_cast<int64_t>(row) * C + (m & ~15)) * a.T + (m & 15);
#pragma unroll
    for (int nb = 0; nb < WNB; ++nb) {
      // Unconditional load (frame clamped into the row; clamped values
      // are never stored), so the prefetch is not serialised.
      const int n = min(n0 + wn * WNB * 16 + nb * 16 + lr, Lv - 1);
      hres[mb][nb] = load_h4_raw<HO>(a.h_in, hbase + static_cast<int64_t>(n) * kHChunk);
    }
  };
  auto load_h = [&]() {
#pragma unroll
    for (int mb = 0; mb < WMB; ++mb) load_h_block(mb);
  };
  if constexpr (kEarlyH) load_h();

  // ------------------------------------------------------------ stage 1
  // Staging unit idx covers frame tfirst + unit_row(idx) and the 16 operand
  // bytes at unit_col(idx) of the chunk row; unit_col(idx) == lg for every u,
  // so each thread stages the same 16 / ES channels of every chunk row.
  constexpr int HV = XH ? 16 / ES / 4 : 1;  // h quads per staging unit
  uint4 xr[XH ? 1 : XU], wr[WU];
  typename HQuad<HO>::T xh[XH ? XU : 1][HV];  // raw h, converted at staging
  // Snake1 parameters (scale[C], h[C]) in LDS: read at staging time
  // rather than held in registers across the matrix work.
  float* P1 = reinterpret_cast<float*>(smem + LDS_T);
  int xch = 0;  // first channel of this thread's staging units (chunk of the last load_x)
  bool xlo = false;  // the last load_x staged a low-term chunk (two terms)
  if constexpr (XH) {
    for (int i = tid; i < C / 4; i += NTH) {
      reinterpret_cast<f4*>(P1)[i] = reinterpret_cast<const f4*>(a.a1_scale)[i];
      reinterpret_cast<f4*>(P1 + C)[i] = reinterpret_cast<const f4*>(a.a1_h)[i];
    }
    __syncthreads();
  }
  auto load_x = [&](int c) {
    if constexpr (XH) {
      const int ch = (TERMS == 2 && c >= NCH ? c - NCH : c) * CH + lg * (16 / ES);
      xch = ch;
      xlo = TERMS == 2 && c >= NCH;
      const int64_t hp = (static_cast<int64_t>(row) * C + (ch & ~15)) * a.T + (ch & 15);
#pragma unroll
      for (int u = 0; u < XU; ++u) {
        const int r = unit_row(tid + u * NTH);
        const int t = tfirst + r;
        const bool in = r < xrows && t >= -a.lb && t < Lv;
#pragma unroll
        for (int v = 0; v < HV; ++v)
          xh[u][v] = in ? load_h4_raw<HO>(a.h_in, hp + static_cast<int64_t>(t) * kHChunk + 4 * v)
                        : typename HQuad<HO>::T{};
      }
      // Residual rows of this chunk's channels, while the X lines are in L2.
      if constexpr (kChunkH) {
#pragma unroll
        for (int mb = 0; mb < WMB; ++mb)
          if ((wm * WMB * 16 + mb * 16) / CH == c) load_h_block(mb);
      }
    } else {
      const unsigned char* xc = xrow + c * xplane;
#pragma unroll
      for (int u = 0; u < XU; ++u) {
        const int idx = tid + u * NTH;
        const int r = unit_row(idx), col = unit_col(idx);
        const int t = tfirst + r;
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (r < xrows && t >= -a.lb && t < Lv)
          v = *reinterpret_cast<const uint4*>(xc + static_cast<int64_t>(t) * kChunkBytes + col * 16);
        xr[u] = v;
      }
    }
  };
  auto load_w = [&](int c, int g) {
#pragma unroll
    for (int u = 0; u < WU; ++u) {
      const int idx = tid + u * NTH;
      const int r = unit_row(idx), col = unit_col(idx);
      const int jj = r / C, m = r - jj * C;
      const int j = g * TG + jj;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (r < WROWS && j < 7)
        v = *reinterpret_cast<const uint4*>(
            w1 + ((static_cast<int64_t>(c) * 7 + j) * C + m) * kChunkBytes + col * 16);
      wr[u] = v;
    }
  };
  auto store_x = [&](unsigned char* Xs) {
#pragma unroll
    for (int u = 0; u < XU; ++u) {
      const int idx = tid + u * NTH;
      const int r = unit_row(idx);
      if (r >= xrows) continue;
      uint4 v;
      if constexpr (XH) {
        // Snake1 in fp32, then the operand dtype; frames outside [-lb, Lv)
        // are the convolution's zero padding.
        // (The padding is applied to the packed operand bits: one select per
        // 32-bit word.)
        const int t = tfirst + r;
        const bool in = t >= -a.lb && t < Lv;
        float y[4 * HV];
#pragma unroll
        for (int q = 0; q < HV; ++q) {
          const f4 ps = *reinterpret_cast<const f4*>(P1 + xch + 4 * q);
          const f4 ph = *reinterpret_cast<const f4*>(P1 + C + xch + 4 * q);
          const f4 xq = h4_to_f4<HO>(xh[u][q]);
#pragma unroll
          for (int e = 0; e < 4; ++e) y[4 * q + e] = snake_f32(xq[e], ps[e], ph[e]);
        }
        if constexpr (TERMS == 2) {
          if (xlo) {
#pragma unroll
            for (int k = 0; k < 4 * HV; ++k) y[k] -= bf16_round(y[k]);
          }
        }
        if constexpr (OP == OP_BF16) {
          v.x = pack_bf16x2(y[0], y[1]);
          v.y = pack_bf16x2(y[2], y[3]);
          v.z = pack_bf16x2(y[4], y[5]);
          v.w = pack_bf16x2(y[6], y[7]);
        } else {
          v = make_uint4(__float_as_uint(y[0]), __float_as_uint(y[1]), __float_as_uint(y[2]),
                         __float_as_uint(y[3]));
        }
        if (!in) v = make_uint4(0u, 0u, 0u, 0u);
        if constexpr (kPair) {  // the low terms into the second half of the buffer
#pragma unroll
          for (int k = 0; k < 4 * HV; ++k) y[k] -= bf16_round(y[k]);
          uint4 vl;
          vl.x = pack_bf16x2(y[0], y[1]);
          vl.y = pack_bf16x2(y[2], y[3]);
          vl.z = pack_bf16x2(y[4], y[5]);
          vl.w = pack_bf16x2(y[6], y[7]);
          if (!in) vl = make_uint4(0u, 0u, 0u, 0u);
          *reinterpret_cast<uint4*>(Xs + XROWS * kRowBytes + lds_off(r, unit_col(idx))) = vl;
        }
      } else {
        v = xr[u];
      }
      *reinterpret_cast<uint4*>(Xs + lds_off(r, unit_col(idx))) = v;
    }
  };
  auto store_w = [&](unsigned char* Ws) {
#pragma unroll
    for (int u = 0; u < WU; ++u) {
      const int idx = tid + u * NTH;
      const int r = unit_row(idx);
      if (r < WROWS) *reinterpret_cast<uint4*>(Ws + lds_off(r, unit_col(idx))) = wr[u];
    }
  };

  // Matrix steps of tap group g from the X tile at xs and the weights at ws.
  auto mma_group = [&](int g, const unsigned char* xs, const unsigned char* ws) {
    const int nt = (g + 1) * TG <= 7 ? TG : 7 - g * TG;  // taps in this group
    const unsigned char* wt = ws + (wm * WMB * 16) * kRowBytes + lane * 16;
    const int xr0 = g * TG * d + wn * WNB * 16 + lr;
    mma_steps<OP, WMB, WNB, TG, false>(
        acc, nt, [&](int jj, int mb) { return wt + (jj * C + mb * 16) * kRowBytes; },
        [&](int jj, int nb) { return xs + lds_off(xr0 + jj * d, lg) + nb * 1024; });
    if constexpr (kPair)  // the same weights against the low-term tile
      mma_steps<OP, WMB, WNB, TG, false>(
          acc, nt, [&](int jj, int mb) { return wt + (jj * C + mb * 16) * kRowBytes; },
          [&](int jj, int nb) { return xs + XROWS * kRowBytes + lds_off(xr0 + jj * d, lg) + nb * 1024; });
  };
  load_x(0);
  load_w(0, 0);
  if constexpr (kDB) {
    // Group p = c * NG + g uses X buffer c & 1 and weight buffer p & 1.  In
    // group p the waves store group p + 1 (loaded during group p - 1) into
    // the other buffers, request group p + 2, and multiply group p; the
    // barrier at its end makes group p + 1 visible and frees group p's
    // buffers for group p + 2.
    store_x(Xs);
    store_w(Ws);
    if (NG > 1) {
      load_w(0, 1);
    } else if (LCH > 1) {
      load_x(1);
      load_w(1, 0);
    }
    __syncthreads();
    for (int c = 0; c < LCH; ++c) {
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const int p = c * NG + g;
        const int c1 = g + 1 < NG ? c : c + 1, g1 = g + 1 < NG ? g + 1 : 0;
        auto stage_next = [&]() {
          if (c1 < LCH) {
            if (g1 == 0) store_x(Xs + (c1 & 1) * XT * kRowBytes);
            store_w(Ws + ((p + 1) & 1) * WROWS * kRowBytes);
            const int c2 = g1 + 1 < NG ? c1 : c1 + 1, g2 = g1 + 1 < NG ? g1 + 1 : 0;
            if (c2 < LCH) {
              if (g2 == 0) load_x(c2);
              load_w(c2, g2);
            }
          }
        };
        if (VOC_RU_PINGPONG && wave >= WAVES_M * WAVES_N / 2) {
          mma_group(g, Xs + (c & 1) * XT * kRowBytes, Ws + (p & 1) * WROWS * kRowBytes);
          stage_next();
        } else {
          stage_next();
          mma_group(g, Xs + (c & 1) * XT * kRowBytes, Ws + (p & 1) * WROWS * kRowBytes);
        }
        __syncthreads();
      }
    }
  } else {
    for (int c = 0; c < LCH; ++c) {
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        if (g == 0) store_x(Xs);
        store_w(Ws);
        __syncthreads();
        if (g + 1 < NG) {
          load_w(c, g + 1);
        } else if (c + 1 < LCH) {
          load_x(c + 1);
          load_w(c + 1, 0);
        }
        mma_group(g, Xs, Ws);
        __syncthreads();
      }
    }
  }

  if constexpr (!kEarlyH && !kChunkH) load_h();

  // Fetch the first conv2 weight chunk while the U epilogue runs.
  uint4 w2r[W2U];
  auto load_w2 = [&](int c) {
#pragma unroll
    for (int u = 0; u < W2U; ++u) {
      const int idx = tid + u * NTH;
      const int r = unit_row(idx), col = unit_col(idx);
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (r < C)
        v = *reinterpret_cast<const uint4*>(
            w2 + (static_cast<int64_t>(c) * C + r) * kChunkBytes + col * 16);
      w2r[u] = v;
    }
  };
  load_w2(0);

  // ------------------------------------------- epilogue 1: U into LDS
#pragma unroll
  for (int mb = 0; mb < WMB; ++mb) {
    const int m = wm * WMB * 16 + mb * 16 + lg * 4;
    const f4 b1 = *reinterpret_cast<const f4*>(a.b1 + m);
    const f4 sc = *reinterpret_cast<const f4*>(a.a2_scale + m);
    const f4 hh = *reinterpret_cast<const f4*>(a.a2_h + m);
    // U rows are frames of one channel chunk; this lane's 4 channels sit in
    // unit (m % CH) * ES / 16 of the row, at byte (m % CH) * ES % 16.
    const int ub = (m % CH) * ES;
    unsigned char* ubase = Us + (m / CH) * BN * kRowBytes + (ub & 15);
#pragma unroll
    for (int nb = 0; nb < WNB; ++nb) {
      const int nl = wn * WNB * 16 + nb * 16 + lr;
      f4 v = acc[mb][nb] + b1;
      v[0] = snake_f32(v[0], sc[0], hh[0]);
      v[1] = snake_f32(v[1], sc[1], hh[1]);
      v[2] = snake_f32(v[2], sc[2], hh[2]);
      v[3] = snake_f32(v[3], sc[3], hh[3]);
      store_op4<OP>(ubase + lds_off(nl, ub >> 4), 0, v);
      if constexpr (TERMS == 2)  // the low terms: chunk rows NCH.. of the U tile
        store_op4<OP>(ubase + NCH * BN * kRowBytes + lds_off(nl, ub >> 4), 0, bf16_lo4(v));
      acc[mb][nb] = f4{0.f, 0.f, 0.f, 0.f};
    }
  }

  // ------------------------------------------------------------ stage 2
  // (Two terms: each conv2 weight chunk c meets U's high-term chunk c and its
  // low-term chunk NCH + c.)
  for (int c = 0; c < NCH; ++c) {
#pragma unroll
    for (int u = 0; u < W2U; ++u) {
      const int idx = tid + u * NTH;
      const int r = unit_row(idx);
      if (r < C) *reinterpret_cast<uint4*>(W2s + lds_off(r, unit_col(idx))) = w2r[u];
    }
    __syncthreads();
    if (c + 1 < NCH) load_w2(c + 1);
    uint4 A[WMB], B[WNB];
#pragma unroll
    for (int mb = 0; mb < WMB; ++mb)
      A[mb] = *reinterpret_cast<const uint4*>(W2s + (wm * WMB * 16 + mb * 16) * kRowBytes + lane * 16);
#pragma unroll
    for (int t = 0; t < TERMS; ++t) {
#pragma unroll
      for (int nb = 0; nb < WNB; ++nb)
        B[nb] = *reinterpret_cast<const uint4*>(
            Us + ((t * NCH + c) * BN + wn * WNB * 16 + nb * 16) * kRowBytes + lane * 16);
#pragma unroll
      for (int mb = 0; mb < WMB; ++mb)
#pragma unroll
        for (int nb = 0; nb < WNB; ++nb) mfma_frag<OP>(A[mb], B[nb], acc[mb][nb]);
    }
    __syncthreads();
  }

  // ----------------------------------- epilogue 2: bias, skip, next Snake
  if constexpr (OP == OP_BF16 && WMB % 2 == 0) {
    // The two 16-row blocks of a 32-channel chunk are finished together and
    // one lane exchange (lane ^ 16) gives each lane 8 contiguous operand
    // channels: each frame's 64-byte operand row is written as four 16-byte
    // stores instead of eight 8-byte half-row pieces.
    typedef uint32_t u4v __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int mp = 0; mp < WMB; mp += 2) {
      const int m = wm * WMB * 16 + mp * 16 + lg * 4;  // first block's rows
      f4 b2[2], sc[2], hh[2], hsc[2], hsh[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        b2[q] = *reinterpret_cast<const f4*>(a.b2 + m + 16 * q);
        sc[q] = hh[q] = hsc[q] = hsh[q] = f4{0.f, 0.f, 0.f, 0.f};
        if (a.s_out) {
          sc[q] = *reinterpret_cast<const f4*>(a.s_scale + m + 16 * q);
          hh[q] = *reinterpret_cast<const f4*>(a.s_h + m + 16 * q);
        }
        if (a.hs_scale) {
          hsc[q] = *reinterpret_cast<const f4*>(a.hs_scale + m + 16 * q);
          hsh[q] = *reinterpret_cast<const f4*>(a.hs_h + m + 16 * q);
        }
      }
      const int mc = m - lg * 4;                       // chunk's first channel
      const int cofs = (lg & 1) * 16 + (lg & 2) * 4;   // this lane's 8 channels
      const int64_t sbase = (static_cast<int64_t>(row) * TERMS * C + mc) * a.T + cofs;
      const int64_t slo = static_cast<int64_t>(C) * a.T;  // low-term planes (two terms)
#pragma unroll
      for (int nb = 0; nb < WNB; ++nb) {
        const int n = n0 + wn * WNB * 16 + nb * 16 + lr;
        const bool ok = n < Lv;
        u4v pk, pl;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int mq = m + 16 * q;
          f4 v = acc[mp + q][nb] + b2[q] + h4_to_f4<HO>(hres[mp + q][nb]);
          if (a.s_out || a.hs_scale) v = round_h4<HO>(v);  // a Snake follows: start from the stored h
          if (a.store_h && ok) {
            f4 hv = v;
            if (a.hs_scale) {
              hv[0] = snake_f32(v[0], hsc[q][0], hsh[q][0]);
              hv[1] = snake_f32(v[1], hsc[q][1], hsh[q][1]);
              hv[2] = snake_f32(v[2], hsc[q][2], hsh[q][2]);
              hv[3] = snake_f32(v[3], hsc[q][3], hsh[q][3]);
            }
            const int64_t hi = (static_cast<int64_t>(row) * C + (mq & ~15)) * a.T + (mq & 15) +
                               static_cast<int64_t>(n) * kHChunk;
            store_h4<HO>(a.h, hi, hv);
          }
          if (a.s_out) {
            f4 sv;
            sv[0] = snake_f32(v[0], sc[q][0], hh[q][0]);
            sv[1] = snake_f32(v[1], sc[q][1], hh[q][1]);
            sv[2] = snake_f32(v[2], sc[q][2], hh[q][2]);
            sv[3] = snake_f32(v[3], sc[q][3], hh[q][3]);
            pk[2 * q] = pack_bf16x2(sv[0], sv[1]);
            pk[2 * q + 1] = pack_bf16x2(sv[2], sv[3]);
            if constexpr (TERMS == 2) {
              const f4 lv = bf16_lo4(sv);
              pl[2 * q] = pack_bf16x2(lv[0], lv[1]);
              pl[2 * q + 1] = pack_bf16x2(lv[2], lv[3]);
            }
          }
        }
        if (a.s_out) {  // uniform: every lane takes part in the exchange
          const bool odd = lg & 1;
          auto exchange = [&](const u4v& p) {
            const uint32_t s0 = __shfl_xor(static_cast<int>(odd ? p[0] : p[2]), 16);
            const uint32_t s1 = __shfl_xor(static_cast<int>(odd ? p[1] : p[3]), 16);
            u4v out;
            if (odd) {
              out[0] = s0; out[1] = s1; out[2] = p[2]; out[3] = p[3];
            } else {
              out[0] = p[0]; out[1] = p[1]; out[2] = s0; out[3] = s1;
            }
            return out;
          };
          const u4v out = exchange(pk);
          if (ok)
            *reinterpret_cast<u4v*>(static_cast<uint16_t*>(a.s_out) + sbase + static_cast<int64_t>(n) * CH) = out;
          if constexpr (TERMS == 2) {
            const u4v outl = exchange(pl);
            if (ok)
              *reinterpret_cast<u4v*>(static_cast<uint16_t*>(a.s_out) + sbase + slo + static_cast<int64_t>(n) * CH) =
                  outl;
          }
        }
      }
    }
  } else {
  #pragma unroll
    for (int mb = 0; mb < WMB; ++mb) {
      const int m = wm * WMB * 16 + mb * 16 + lg * 4;
      const f4 b2 = *reinterpret_cast<const f4*>(a.b2 + m);
      f4 sc = f4{0.f, 0.f, 0.f, 0.f}, hh = f4{0.f, 0.f, 0.f, 0.f};
      if (a.s_out) {
        sc = *reinterpret_cast<const f4*>(a.s_scale + m);
        hh = *reinterpret_cast<const f4*>(a.s_h + m);
      }
      f4 hsc = f4{0.f, 0.f, 0.f, 0.f}, hsh = f4{0.f, 0.f, 0.f, 0.f};
      if (a.hs_scale) {
        hsc = *reinterpret_cast<const f4*>(a.hs_scale + m);
        hsh = *reinterpret_cast<const f4*>(a.hs_h + m);
      }
      const int64_t hbase = (static_cast<int64_t>(row) * C + (m & ~15)) * a.T + (m & 15);
      const int64_t sbase = (static_cast<int64_t>(row) * TERMS * C + (m / CH) * CH) * a.T + (m % CH);
  #pragma unroll
      for (int nb = 0; nb < WNB; ++nb) {
        const int n = n0 + wn * WNB * 16 + nb * 16 + lr;
        if (n >= Lv) continue;
        const int64_t hidx = hbase + static_cast<int64_t>(n) * kHChunk;
        f4 v = acc[mb][nb] + b2 + h4_to_f4<HO>(hres[mb][nb]);
        if (a.s_out || a.hs_scale) v = round_h4<HO>(v);  // a Snake follows: start from the stored h
        f4 hv = v;
        if (a.hs_scale) {
          hv[0] = snake_f32(v[0], hsc[0], hsh[0]);
          hv[1] = snake_f32(v[1], hsc[1], hsh[1]);
          hv[2] = snake_f32(v[2], hsc[2], hsh[2]);
          hv[3] = snake_f32(v[3], hsc[3], hsh[3]);
        }
        if (a.store_h) store_h4<HO>(a.h, hidx, hv);
        if (a.s_out) {
          v[0] = snake_f32(v[0], sc[0], hh[0]);
          v[1] = snake_f32(v[1], sc[1], hh[1]);
          v[2] = snake_f32(v[2], sc[2], hh[2]);
          v[3] = snake_f32(v[3], sc[3], hh[3]);
          store_op4<OP>(a.s_out, sbase + static_cast<int64_t>(n) * CH, v);
          if constexpr (TERMS == 2)
            store_op4<OP>(a.s_out, sbase + static_cast<int64_t>(C) * a.T + static_cast<int64_t>(n) * CH,
                          bf16_lo4(v));
        }
      }
    }
  }
}

// Instances: channel width C -> {m-blocks per wave, n-blocks, waves M, waves N,
// taps per group, waves per SIMD}.
// Only widths where one fused launch beats the conv1 + conv2 pair on MI355X
// (per-layer kernel traces): at C >= 256 the whole-C tile leaves too few
// frames per workgroup (LDS holds U for all C), and the pair is faster (a
// 256-channel eight-wave tile measured 1040 us per unit against 1000 us for
// the pair on the batched bf16 windows).
// Per dtype and width: a large-frame tile, the fastest in per-layer traces of
// the full workloads on MI355X, and a half-frame tile for launches too short
// to give the large one two workgroups per CU.  The 64-channel large tiles
// are sized for occupancy: at most 128 VGPRs give 16 waves per CU, whose
// staging, Snake and epilogue phases then overlap other workgroups' matrix
// phases.  fp32: four four-wave workgroups of 128 frames (4 % faster per unit
// than 256 frames at two workgroups); bf16: two eight-wave workgroups of 256
// frames, one stage-1 buffer (22 % faster than 256 frames at one four-wave
// workgroup pair, 12 % faster than four 128-frame workgroups).  Overridable
// at build time for sweeps.
#ifndef VOC_F32_RU64
#define VOC_F32_RU64 4, 2, 1, 4, 1, 4
#endif
#ifndef VOC_F32_RU96
#define VOC_F32_RU96 6, 2, 1, 4, 7, 2
#endif
#ifndef VOC_F32_RU128
#define VOC_F32_RU128 4, 4, 2, 2, 4, 2
#endif
#ifndef VOC_BF_RU64
#define VOC_BF_RU64 2, 4, 2, 4, 2, 4
#endif
#ifndef VOC_BF_RU96
#define VOC_BF_RU96 6, 4, 1, 4, 7, 2
#endif
#ifndef VOC_BF_RU128
#define VOC_BF_RU128 4, 4, 2, 4, 4, 1
#endif
#ifndef VOC_BF_RU192
#define VOC_BF_RU192 3, 4, 4, 2, 4, 1
#endif
#define VOC_RU_(...) VOC_RU(__VA_ARGS__)
template <int OP>
static hipError_t launch_ru(const ResUnitArgs& a, bool big, hipStream_t s, int* bn) {
  if (a.terms < 0 || a.terms > 2 || (a.terms == 2 && OP != OP_BF16)) return hipErrorInvalidValue;
  // With two-term operands the 96-channel large tile's U tile (2 x 3 chunks x
  // 256 frames) would leave one workgroup per CU: the half-frame tile serves.
  if (a.terms == 2 && a.C == 96) big = false;
#define VOC_RU_T(A, B, WM, WN, TGV, MB, TM)                                                     \
  if (a.x_from_h)                                                                                 \
    hipLaunchKernelGGL((res_unit_kernel<OP, A, B, WM, WN, TGV, true, MB, TM>),                    \
                       dim3(a.n_tiles * a.rows), dim3(64 * WM * WN), 0, s, a);                    \
  else                                                                                            \
    hipLaunchKernelGGL((res_unit_kernel<OP, A, B, WM, WN, TGV, false, MB, TM>),                   \
                       dim3(a.n_tiles * a.rows), dim3(64 * WM * WN), 0, s, a);
#define VOC_RU(CW, BIG, A, B, WM, WN, TGV, MB)                                                    \
  if (a.C == CW && big == BIG) {                                                                  \
    *bn = WN * B * 16;                                                                            \
    if (a.n_tiles <= 0) return hipSuccess;                                                        \
    if constexpr (OP == OP_BF16) {                                                                \
      if (a.terms == 2) {                                                                         \
        VOC_RU_T(A, B, WM, WN, TGV, MB, 2)                                                        \
        return hipGetLastError();                                                                 \
      }                                                                                           \
    }                                                                                             \
    VOC_RU_T(A, B, WM, WN, TGV, MB, 1)                                                            \
    return hipGetLastError();                                                                     \
  }
// A tile used with two-term operands only.
#define VOC_RU2(CW, BIG, A, B, WM, WN, TGV, MB)                                                   \
  if constexpr (OP == OP_BF16) {                                                                  \
    if (a.C == CW && big == BIG && a.terms == 2) {                                                \
      *bn = WN * B * 16;                                                                          \
      if (a.n_tiles <= 0) return hipSuccess;                                                      \
      VOC_RU_T(A, B, WM, WN, TGV, MB, 2)                                                          \
      return hipGetLastError();                                                                   \
    }                                                                                             \
  }
// A tile used with one-term operands only.
#define VOC_RU1(CW, BIG, A, B, WM, WN, TGV, MB)                                                   \
  if (a.C == CW && big == BIG && a.terms != 2) {                                                  \
    *bn = WN * B * 16;                                                                            \
    if (a.n_tiles <= 0) return hipSuccess;                                                        \
    VOC_RU_T(A, B, WM, WN, TGV, MB, 1)                                                            \
    return hipGetLastError();                                                                     \
  }
#define VOC_RU1_(...) VOC_RU1(__VA_ARGS__)
#define VOC_RU2_(...) VOC_RU2(__VA_ARGS__)
  if constexpr (OP == OP_BF16) {
    VOC_RU_(64, true, VOC_BF_RU64)
    VOC_RU(64, false, 4, 2, 1, 4, 7, 2)
    VOC_RU1_(96, true, VOC_BF_RU96)
#ifndef VOC_BF_RU96_T2
#define VOC_BF_RU96_T2 6, 2, 1, 4, 2, 2
#endif
    VOC_RU2_(96, false, VOC_BF_RU96_T2)
    VOC_RU(96, false, 6, 2, 1, 4, 7, 2)
    VOC_RU_(128, true, VOC_BF_RU128)
    VOC_RU(128, false, 4, 4, 2, 2, 4, 2)
    VOC_RU_(192, true, VOC_BF_RU192)
    VOC_RU(192, false, 3, 4, 4, 1, 2, 2)
  } else {
    VOC_RU(16, false, 1, 4, 1, 4, 7, 2)
    VOC_RU(32, false, 2, 2, 1, 4, 7, 2)
    VOC_RU_(64, true, VOC_F32_RU64)
    VOC_RU(64, false, 4, 2, 1, 4, 7, 2)
    VOC_RU_(96, true, VOC_F32_RU96)
    VOC_RU(96, false, 6, 2, 1, 4, 7, 2)
    VOC_RU_(128, true, VOC_F32_RU128)
    VOC_RU(128, false, 4, 2, 2, 2, 4, 2)
  }
#undef VOC_RU
#undef VOC_RU_
#undef VOC_RU1
#undef VOC_RU1_
#undef VOC_RU2
#undef VOC_RU2_
#undef VOC_RU_T
  return hipErrorInvalidValue;
}

int res_unit_tile(int op, int C, bool big, int terms) {
  int bn = 0;
  ResUnitArgs probe{};
  probe.C = C;
  probe.terms = terms;
  probe.n_tiles = 0;
  const hipError_t e = op == OP_F32 ? launch_ru<OP_F32>(probe, big, nullptr, &bn)
                                    : launch_ru<OP_BF16>(probe, big, nullptr, &bn);
  return e == hipSuccess ? bn : 0;
}

hipError_t launch_res_unit(int op, const ResUnitArgs& a, bool big, hipStream_t s) {
  int bn = 0;
  return op == OP_F32 ? launch_ru<OP_F32>(a, big, s, &bn) : launch_ru<OP_BF16>(a, big, s, &bn);
}

}  // namespace voc
