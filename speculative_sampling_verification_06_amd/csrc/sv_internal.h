// sv_internal.h - declarations shared by the library's own HIP sources (not part of the C ABI).
#ifndef SV_INTERNAL_H
#define SV_INTERNAL_H

#include <stddef.h>
#include <stdint.h>

#include "spec_verify.h"

// The verify step with separate storage types for the target and draft logits
// (SV_F32 / SV_BF16 each); same arguments and errors as spec_verify otherwise.
// With check_only != 0 it runs the host checks and launches nothing.
int sv_verify_mixed(const void* target, const void* draft, const int32_t* tokens, const float* uniforms,
                    float T, const uint8_t* greedy, int32_t B, int32_t K, int32_t V, int32_t dtt,
                    int32_t dtd, int32_t* acc, int32_t* out, const sv_diag* diag, void* ws,
                    size_t ws_bytes, void* stream, int check_only);

// Launch bookkeeping of every entry point: sv_launch_begin() clears an error a
// caller's earlier HIP call may have left (it is not this call's failure);
// sv_launch_status() after the launches returns SV_OK or SV_ELAUNCH and keeps
// the HIP error code for sv_last_hip_error().
void sv_launch_begin(void);
int sv_launch_status(void);

#endif
