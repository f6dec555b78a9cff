// Kernels of table row 1 (see mg_table.h).
#include "mg_launch.h"

MG_DEFINE_ROW(1, Cfg1, Fast1)
