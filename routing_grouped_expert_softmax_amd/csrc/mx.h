// mx.h — internal MXFP8 helpers shared by mx.hip and gemm_mx.hip.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

// Rowwise quantisation of a bf16 [rows][cols] matrix (cols % 32 == 0):
// codes [rows][cols], scales [rows][cols/32].
hipError_t mx_quantize_rows(const void* src, int rows, int cols, uint8_t* codes, uint8_t* scales,
                            hipStream_t s);
// Column-block quantisation with row groups (offsets[G+1] on the device, or
// `urows` rows per group when offsets is null), transposed output
// codes [cols][kpad_ld], scales [cols][kpad_ld/32]; group g owns K positions
// starting at the exclusive scan of roundup(n_g, 128).
hipError_t mx_quantize_cols(const void* src, int rows, int cols, const int32_t* offsets, int urows,
                            int groups, uint8_t* codes, uint8_t* scales, int kpad_ld,
                            hipStream_t s);
// mx_quantize_cols plus, from the same read, the rowwise layout of the rows
// the groups cover (rcodes [rows][cols], rscales [rows][cols/32]), equal to
// mx_quantize_rows of those rows byte for byte.
hipError_t mx_quantize_both(const void* src, int rows, int cols, const int32_t* offsets, int urows,
                            int groups, uint8_t* codes, uint8_t* scales, int kpad_ld,
                            uint8_t* rcodes, uint8_t* rscales, hipStream_t s);
// A weight pack's regions: the forward layouts (f*: Wg, Wu codes
// [F][E*d], Wd codes [d][E*F], blocks along each expert matrix's rows) and
// the backward layouts (b*: Wg, Wu codes [E*d][F], Wd codes [E*F][d], blocks
// along the columns), each with its scale bytes.
struct MxWeights {
  const uint8_t *fgq, *fgs, *fuq, *fus, *fdq, *fds;
  const uint8_t *bgq, *bgs, *buq, *bus, *bdq, *bds;
};
// Upper bound of the padded K of a column-quantised operand (a multiple of
// 128 is the caller's leading dimension).
long long mx_kpad_bound(int rows, int groups);
