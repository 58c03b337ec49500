// et_gemm.hpp -- bf16 MFMA tiles for the GEMM tasks (gfx950, wave64).
//
// Both tiles accumulate in fp32 with v_mfma_f32_16x16x32_bf16 and take the
// weights (B) K-contiguous ([N, K]) straight from global memory into VGPRs in
// MFMA operand layout: lane (j = lane%16, g = lane/16) of a 16-column group
// holds column j.  For one 128-element K-block, lane group g loads the 64
// contiguous bytes [64g, 64g + 64) of its row as four 16-byte loads, so four
// lanes cover 256 contiguous bytes of a weight row: whole cache lines of the
// weight stream.  MFMA step s (0..3) consumes elements 32g + 8s .. 32g + 8s + 7
// of both operands; the reduction runs over all 128 elements, so this K
// permutation is harmless as long as A uses the same one.
//
// StreamTile (few rows, the decode regime): A also streams from global memory
// into VGPRs (lane (i = lane%16, g) holds row i).  The four waves split the
// tile as WK (K-split) x 4/WK (N-split); with WK > 1 wave wk consumes K-blocks
// wk, wk + WK, ... and the partial tiles are summed through LDS.  Loads run PD
// K-blocks ahead of the MFMAs (a register ring), keeping enough bytes in
// flight per CU to stream weights at HBM rate.
//
// RingTile (many rows, the MFMA-bound regime): 16*MT rows x 256 columns, the
// four waves splitting the columns (64 each, four 16-column groups).  Both
// operands of a 64-element K-stage are copied straight from global memory
// into LDS by the buffer unit (16 bytes per lane, no VGPR staging), into a
// ring of three stages, so two stages are always in flight while the MFMAs
// consume the third.  Rows are 128 bytes with the 16-byte chunks XOR-swizzled
// by (row / 2) mod 8: the copy writes whole rows contiguously and the 16
// rows one ds_read_b128 reads fall into 16 disjoint 4-bank groups.
//
// In both, rows outside the valid range use an out-of-range buffer offset and
// read as zeros, and A can be read agent-coherently (COH) when it was written
// earlier in the same launch.  gate(round) runs uniformly on all waves before
// the A loads of a round (gate(0) always runs and may fill the row table); the
// weights of the first rounds are requested before gate(0), so the weight
// stream starts before the activations it multiplies are ready (the prefetch
// rewrite of Event Tensor notes, section "ETC 编译流程", and the weight
// prefetch of section "端到端低 batch serving").
#pragma once

#include "et_device.hpp"

namespace et {

template <int MT, int NB, int WK, int PD, bool COH>
struct StreamTile {
  static constexpr int kRedFloats = WK > 1 ? 4 * MT * NB * 4 * 64 : 1;   // LDS floats
  static constexpr int kLdsBytes = kRedFloats * 4;   // reduction scratch
  static constexpr int kStageBytes = 0;                // no LDS ring

  // acc[mt][nb]: rows 16*mt + 4*(lane/16) + r, column 16*nb + lane%16 of this
  // wave's column group (for WK > 1: summed over the K-split waves).
  f32x4 acc[MT][NB];

  template <class Gate>
  __device__ __forceinline__ bool run(Rsrc ra, const uint32_t* a_row_off /* [16*MT], LDS */,
                                      const Rsrc* rb, const uint32_t* b_row_off /* [NB] */,
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
          for (int s = 0; s < 4; ++s) abuf[p][m][s] = ld16x<COH>(ra, aoff[m] + o + 16u * s);
      }
    };

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

#define ET_LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

// 16 bytes per lane, global -> LDS at lds_base + 16 * lane (sc1 when COH).
template <bool COH>
__device__ __forceinline__ void dma16(Rsrc r, void* lds_base, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, ET_LDS_PTR(lds_base), 16, voff, 0, 0, COH ? 16 : 0);
}

// Workgroup barrier that waits for this wave's LDS accesses only (the
// compiler's __syncthreads also waits for every outstanding global store).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Wait until at most N of this wave's memory loads are outstanding, then the
// workgroup barrier (a compiler memory barrier too).
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"i"(N) : "memory");
}

template <int MT, bool COH>
struct RingTile {
  static constexpr int kRows = 16 * MT;                   // A rows
  static constexpr int kCols = 256;                       // B rows = output columns
  static constexpr int kStageBytes = (kRows + kCols) * 128;
  static constexpr int kLdsBytes = 0;                     // besides the three ring slots
  static constexpr int kLA = kRows / 32;                  // A copies per wave per stage
  static constexpr int kLB = 8;                           // B copies per wave per stage
  static constexpr int kL = kLA + kLB;

  f32x4 acc[MT][4];

  // rb[n] / b_row0[n]: buffer and byte offset of the first row (output
  // column) of this wave's 16-column group n; rows are b_stride bytes apart.
  // s0, s1, s2: the three ring slots, three distinct __shared__ arrays of
  // kStageBytes each -- distinct objects let the compiler wait only for the
  // copies into the slot being read, so two stages stay in flight.
  // mv: 16-row groups holding valid rows (1..MT); the MFMAs of the others
  // are skipped (their rows read as zeros and their results are not stored).
  template <class Gate>
  __device__ __forceinline__ bool run(Rsrc ra, const uint32_t* a_row_off /* [kRows], LDS */,
                                      const Rsrc* rb, const uint32_t* b_row0, uint32_t b_stride,
                                      int K, Gate gate, unsigned char* s0, unsigned char* s1,
                                      unsigned char* s2, int mv = MT) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nks = K / 64;
    const int crow = lane >> 3, cpos = lane & 7;           // this lane's row / chunk in a copy
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int n = 0; n < 4; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};

    // B copies: wave-local rows 8q + crow (group q / 2); logical chunk of this
    // lane's physical slot cpos is cpos ^ ((row / 2) mod 8)
    uint32_t boff[kLB];
#pragma unroll
    for (int q = 0; q < kLB; ++q) {
      const int j = 8 * (q & 1) + crow;                    // row inside group q / 2
      const int c = cpos ^ ((j >> 1) & 7);
      boff[q] = b_row0[q >> 1] + (uint32_t)j * b_stride + 16u * c;
    }
    auto issue_b = [&](int ks, unsigned char* slot) {
      unsigned char* dst = slot + kRows * 128 + wave * 64 * 128;
#pragma unroll
      for (int q = 0; q < kLB; ++q) dma16<false>(rb[q >> 1], dst + q * 1024, boff[q] + ks * 128u);
    };
    uint32_t aoff[kLA];
    auto issue_a = [&](int ks, unsigned char* slot) {
#pragma unroll
      for (int u = 0; u < kLA; ++u) dma16<COH>(ra, slot + (wave + 4 * u) * 1024, aoff[u] + ks * 128u);
    };

    issue_b(0, s0);
    if (nks > 1) issue_b(1, s1);
    if (!gate(0)) {
      wait_vm_barrier<0>();
      return false;
    }
#pragma unroll
    for (int u = 0; u < kLA; ++u) {
      const int row = 8 * (wave + 4 * u) + crow;
      const uint32_t base = a_row_off[row];
      aoff[u] = base == kOOB ? kOOB : base + 16u * (uint32_t)(cpos ^ ((row >> 1) & 7));
    }
    issue_a(0, s0);
    if (nks > 1) issue_a(1, s1);

    // fragment read offsets: row (lane % 16) of each 16-row group, logical
    // chunk 4s + g -> physical chunk (4s + g) ^ ((lane % 16) / 2 mod 8)
    const int fi = lane & 15, fg = lane >> 4;
    uint32_t foff[2];
#pragma unroll
    for (int s2i = 0; s2i < 2; ++s2i)
      foff[s2i] = (uint32_t)fi * 128u + 16u * (uint32_t)((4 * s2i + fg) ^ ((fi >> 1) & 7));

    // one stage: wait for slot `cur` (this wave's copies, then the barrier for
    // everyone's), refill slot `nxt2` (read two stages ago) with stage ks + 2,
    // then the MFMAs of stage ks
    auto step = [&](int ks, const unsigned char* cur, unsigned char* nxt2) {
      if (ks >= nks) return;
      if (ks == 0 || ks + 1 >= nks)
        wait_vm_barrier<0>();
      else
        wait_vm_barrier<kL>();      // stage ks + 1 may still be in flight
      if (ks + 2 < nks) {
        issue_b(ks + 2, nxt2);
        issue_a(ks + 2, nxt2);
      }
      const unsigned char* sb = cur + kRows * 128 + wave * 64 * 128;
      // each 32-element K-step reads all of its fragments first, then runs
      // its MFMAs (the LDS latency is paid once per K-step); 32-row halves
      // beyond the valid rows are skipped
#pragma unroll
      for (int s2i = 0; s2i < 2; ++s2i) {
        i32x4 bf[4], af[MT];
#pragma unroll
        for (int n = 0; n < 4; ++n)
          bf[n] = *reinterpret_cast<const i32x4*>(sb + n * 16 * 128 + foff[s2i]);
#pragma unroll
        for (int m = 0; m < MT; m += 2)
          if (m < mv) {
            af[m] = *reinterpret_cast<const i32x4*>(cur + m * 16 * 128 + foff[s2i]);
            af[m + 1] = *reinterpret_cast<const i32x4*>(cur + (m + 1) * 16 * 128 + foff[s2i]);
          }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int m = 0; m < MT; m += 2)
          if (m < mv) {
#pragma unroll
            for (int n = 0; n < 4; ++n) {
              acc[m][n] = mfma16(af[m], bf[n], acc[m][n]);
              acc[m + 1][n] = mfma16(af[m + 1], bf[n], acc[m + 1][n]);
            }
          }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    for (int ks = 0; ks < nks; ks += 3) {
      step(ks, s0, s2);
      step(ks + 1, s1, s0);
      step(ks + 2, s2, s1);
    }
    wait_vm_barrier<0>();            // the ring may be refilled by the next task
    return true;
  }
};

}  // namespace et
