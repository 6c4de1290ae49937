// qgemv_internal.h -- declarations shared by the host-only and the HIP sources of the library.
#pragma once

#include <stdint.h>

#include "../../include/qgemv.h"

// Shape checks common to qgemv_packed_size / qgemv_repack / qgemv_create.
int qgemv_validate_shape(const qgemv_weights* w);

// Record the hipError_t of a failed runtime call for qgemv_last_hip_error().
void qgemv_set_hip_error(int e);
