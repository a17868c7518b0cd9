// Matrix-core (MFMA, gfx950) kernels of the hot path.
#pragma once

#include "common.h"
