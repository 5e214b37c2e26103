// Arguments and launchers of the 4-bit-weight sparse MLP (k_w4.hip); the
// stored format is defined in include/dv.h (dv_quantize_w4).
#pragma once

#include "dv_internal.h"

namespace dv {

struct W4RowArgs {            // fc1 over selected rows, batch of one
    const float* y;           // [d]
    int d;
    const uint8_t* q;         // [w_rows][d / 2] codes
    const half_t* s;          // [w_rows][d / 128] scales
    const half_t* bias;       // [w_rows]
    const int32_t* idx;       // [n_max] rows, or NULL for 0..n_max-1
    int n_max;
    const int32_t* n_dev;     // rows actually used (<= n_max), or NULL
    int w_rows;
    float* out;               // [n_max] ReLU activations
};

struct W4AxpyArgs {           // fc2 gather-AXPY partials, batch of one
    const uint8_t* q;         // [w_rows][d / 2]
    const half_t* s;          // [w_rows][d / 128]
    int d, w_rows, rows;
    const int32_t* n_rows_dev;
    const int32_t* idx;       // [rows], or NULL
    const float* coef;        // [rows]
    int skip_zero;
    float* partial;           // [w4_axpy_groups(rows)][d]
    int32_t* rows_read;       // incremented by the rows read, or NULL
};

}  // namespace dv

namespace dvh {

dv_status launch_quant_w4(const void* w, int rows, int cols, uint8_t* q, void* s, hipStream_t st);
int w4_chunks_per_lane(int d);
dv_status launch_rowdot_w4(const dv::W4RowArgs& a, hipStream_t s);
int w4_axpy_groups(int rows);
dv_status launch_axpy_w4(const dv::W4AxpyArgs& a, hipStream_t s);
// the gather-AXPY's finalize: out = residual + bias + sum of n_groups partials (k_axpy.hip)
dv_status launch_axpy_finalize(const float* partial, int n_groups, int B, int d, const void* bias, int bias_wdt,
                               const float* residual, float* out, hipStream_t s);

}  // namespace dvh
