// et_gemm.hpp -- bf16 MFMA tile for the GEMM tasks (gfx950, wave64).
//
// One task computes a (16*MT) x (16*NB_per_wave*waves_n) output tile with
// fp32 accumulation using v_mfma_f32_16x16x32_bf16.  Both operands stream
// straight from global memory into VGPRs in MFMA operand layout:
//   A (activations, row-major [rows, K])      lane (i = lane%16, g = lane/16)
//   B (weights, K-contiguous [N, K])          lane (j = lane%16, g = lane/16)
// For one 128-element K-block, lane group g loads the 64 contiguous bytes
// [64g, 64g+64) of its row (four 16-byte loads), so four lanes cover 256
// contiguous bytes of a row: whole cache lines of the weight stream.  MFMA step
// s (0..3) consumes elements 32g + 8s .. 32g + 8s + 7 from both operands; the
// reduction is over all 128 elements, so this K permutation is harmless as
// long as A and B use the same one.
//
// The four waves of a workgroup split the tile as WK (K-split) x 4/WK (N-split).
// With WK > 1, wave wk consumes K-blocks wk, wk + WK, ... and the partial
// accumulators are summed through LDS at the end.  Loads run PD K-blocks
// ahead of the MFMAs (a register ring), which keeps enough bytes in flight per
// CU to stream weights at HBM rate.  Rows outside the tile's valid range use
// an out-of-range buffer offset and read as zeros.
//
// Event-gated A: the caller's gate(round) hook runs (uniformly on all waves)
// before the A loads of each round of WK K-blocks (gate(0) always runs and may
// fill the row-offset table of A); weights for the first PD
// rounds are issued before the first gate, so the weight stream starts before
// the activations it multiplies are ready (the prefetch rewrite of Event
// Tensor notes, section "ETC 编译流程", and the weight prefetch of section
// "端到端低 batch serving").
#pragma once

#include "et_device.hpp"

namespace et {

template <int MT, int NB, int WK, int PD>
struct StreamTile {
  static constexpr int kWavesN = 4 / WK;
  static constexpr int kRedFloats = WK > 1 ? 4 * MT * NB * 4 * 64 : 1;   // LDS floats

  // acc[mt][nb] holds rows 16*mt + 4*(lane/16) + r, column 16*nb + lane%16 of
  // this wave's column group after run() (for WK > 1: summed over waves and
  // valid in every wave of the column group).
  f32x4 acc[MT][NB];

  template <class Gate>
  __device__ __forceinline__ bool run(Rsrc ra, const uint32_t* a_row_off /* [16*MT], LDS */,
                                      const Rsrc* rb, const uint32_t* b_row_off /* [NB] per lane */,
                                      int nkb, Gate gate, float* red /* LDS kRedFloats */) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wk = wave % WK;
    const uint32_t kg = (uint32_t)(lane >> 4) * 64u;
    uint32_t aoff[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int n = 0; n < NB; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int rounds = (nkb + WK - 1) / WK;
    i32x4 abuf[PD][MT][4];
    i32x4 bbuf[PD][NB][4];

    auto load_b = [&](int p, int round) {
      const int kb = round * WK + wk;
      if (round < rounds && kb < nkb) {
        const uint32_t o = (uint32_t)kb * 256u + kg;
#pragma unroll
        for (int n = 0; n < NB; ++n)
#pragma unroll
          for (int s = 0; s < 4; ++s) bbuf[p][n][s] = ld16(rb[n], b_row_off[n] + o + 16u * s);
      }
    };
    auto load_a = [&](int p, int round) {
      const int kb = round * WK + wk;
      if (round < rounds && kb < nkb) {
        const uint32_t o = (uint32_t)kb * 256u + kg;
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
          for (int s = 0; s < 4; ++s) abuf[p][m][s] = ld16(ra, aoff[m] + o + 16u * s);
      }
    };

    // weights first, then (after the gate) activations.  gate(0) may fill
    // a_row_off (it is read only after gate(0) returns).
#pragma unroll
    for (int p = 0; p < PD; ++p) load_b(p, p);
    if (!gate(0)) return false;
#pragma unroll
    for (int m = 0; m < MT; ++m) aoff[m] = a_row_off[16 * m + (lane & 15)];
    load_a(0, 0);
#pragma unroll
    for (int p = 1; p < PD; ++p) {
      if (p < rounds && !gate(p)) return false;
      load_a(p, p);
    }

    for (int j = 0; j < rounds; j += PD) {
#pragma unroll
      for (int p = 0; p < PD; ++p) {
        const int round = j + p;
        const int kb = round * WK + wk;
        if (round < rounds && kb < nkb) {
#pragma unroll
          for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
              for (int n = 0; n < NB; ++n) acc[m][n] = mfma16(abuf[p][m][s], bbuf[p][n][s], acc[m][n]);
        }
        const int nxt = round + PD;
        load_b(p, nxt);
        if (nxt < rounds && !gate(nxt)) return false;
        load_a(p, nxt);
      }
    }

    if (WK > 1) {
      // sum the WK partial tiles of each column group through LDS
      const int wn = wave / WK;
      __syncthreads();
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int n = 0; n < NB; ++n)
#pragma unroll
          for (int r = 0; r < 4; ++r) red[(((wave * MT + m) * NB + n) * 4 + r) * 64 + lane] = acc[m][n][r];
      __syncthreads();
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int n = 0; n < NB; ++n)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float v = 0.f;
#pragma unroll
            for (int q = 0; q < WK; ++q) v += red[((((wn * WK + q) * MT + m) * NB + n) * 4 + r) * 64 + lane];
            acc[m][n][r] = v;
          }
      __syncthreads();
    }
    return true;
  }
};

}  // namespace et
