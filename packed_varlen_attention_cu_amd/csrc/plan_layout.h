// Internal helpers shared by the planner and the kernel launchers.
#pragma once
#include <cstddef>
#include <cstdint>

#include "libra.h"

namespace libra {

// Checksum stored in libra_plan_info::checksum (computed with that field as 0).
uint64_t plan_checksum(const void *plan, size_t bytes);

// Copy the header of a host plan and check its magic and version.
libra_status plan_header(const void *plan, libra_plan_info *out);

}  // namespace libra
